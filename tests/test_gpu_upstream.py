"""GPU parity of the upstream projections (mla_project_down, mla_absorb_from_latent)
against the CPU oracle, at DeepSeek-V3 widths (d_model 7168, d_cq 1536).

The library accumulates in float32 and the oracle in float64; each projection is
then rounded once to bf16.  Where the two sums straddle a bf16 rounding boundary
the stored values differ by one unit in the last place, so the checks are: every
element within a small number of ulps of the exact value; every pool byte
outside the rows the oracle writes still holding the poison, bit for bit; and
the written byte set equal to the oracle's.  All calls go through the C ABI."""
import numpy as np
import pytest
import torch

import mla_synth as S
from oracle import mla_oracle as O
from tests import _util as U

pytestmark = pytest.mark.gpu

V3 = S.WORKLOADS["v3_bs64_ctx8k"]
# float32 accumulation of a 7168-long dot product of O(1) terms moves the value
# before its bf16 rounding by up to about 1e-5 (a few times sqrt(448 k-steps) x
# 2^-24); near zero that is more than a bf16 ulp of the result
ACC_ABS = 2e-5


def _assert_rotated_close(g, e, what, abs_tol=ACC_ABS):
    """Rotated pairs whose raw value (a bf16 projection) may have rounded the other
    way on one side: the raw elements differ by at most one ulp of the pair's norm
    n (u = 2^(floor(log2 n) - 7)), the rotation keeps that difference (at most
    sqrt(2) u) and each side's final rounding adds at most u / 2: 2.5 u in all."""
    n = np.sqrt(e[..., 0::2] ** 2 + e[..., 1::2] ** 2)
    u = np.repeat(np.exp2(np.floor(np.log2(np.maximum(n, 1e-30))) - 7), 2, axis=-1)
    ratio = np.maximum(np.abs(g - e) - abs_tol, 0.0) / u
    assert np.all(ratio <= 2.5), f"{what}: {int((ratio > 2.5).sum())} elements beyond 2.5 u (worst {ratio.max():.2f})"


def _bf16_pool_values(pool_u8: np.ndarray, n_blocks: int, block_size: int, width: int) -> np.ndarray:
    bits = pool_u8.view(np.uint16).reshape(n_blocks, block_size, width)
    return O.bf16_bits_to_f64(bits)


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("lens,d_cq", [([100, 37], 1536), ([64] * 4, 1536), ([1], 1536), ([70, 5], 0)])
def test_project_down_matches_oracle(cache_dtype, lens, d_cq, cuda_device):
    import mla_latent_kv_23_amd as M
    w = V3.replace(cache_dtype=cache_dtype)
    inp = S.make_inputs(w, 810 + len(lens), seqlens=torch.tensor(lens, dtype=torch.int32))
    T = int(sum(lens))
    up = S.make_upstream_inputs(w, 811, T, d_cq=max(d_cq, 16))
    w_down = up["w_down"] if d_cq > 0 else up["w_down"][up["d_cq"]:].contiguous()
    U.say(f"[project_down] cache={cache_dtype} lens={lens} d_cq={d_cq}")
    d = U.dims_of(w)
    dev = cuda_device
    bb = M.cache_block_bytes(d)
    pool = torch.full((inp["n_blocks"] * bb,), 0xA5, dtype=torch.uint8, device=dev)
    c_q = M.project_down(d, up["h"].to(dev), w_down.to(dev), d_cq, inp["tok_seq"].to(dev), inp["tok_pos"].to(dev),
                         inp["block_table"].to(dev), pool)
    # the same call into a pool poisoned with another byte: the bytes the library writes
    # are those where the two pools agree
    pool_5a = torch.full((inp["n_blocks"] * bb,), 0x5A, dtype=torch.uint8, device=dev)
    M.project_down(d, up["h"].to(dev), w_down.to(dev), d_cq, inp["tok_seq"].to(dev), inp["tok_pos"].to(dev),
                   inp["block_table"].to(dev), pool_5a)
    torch.cuda.synchronize()
    h64, wd64 = up["h"].double().numpy(), w_down.double().numpy()
    cq_x, ckv_x, kr_x = O.project_down(h64, wd64, d_cq, w.d_c, w.d_rope, out_dtype=None)
    if d_cq > 0:
        g = c_q.double().cpu().numpy()
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(cq_x), 1e-30))) - 7)
        assert np.all(np.abs(g - cq_x) <= ulp + ACC_ABS), "c_q beyond one ulp"
    # expected pool from the oracle's projections (R17: rounded once to bf16), then the append
    _, ckv_b, kr_b = O.project_down(h64, wd64, d_cq, w.d_c, w.d_rope)
    want = O.append_expected_pool(np.full(inp["n_blocks"] * bb, 0xA5, dtype=np.uint8), ckv_b, kr_b,
                                  inp["tok_seq"].numpy(), inp["tok_pos"].numpy(), inp["block_table"].numpy(),
                                  block_size=w.block_size, d_c=w.d_c, d_rope=w.d_rope, cache_dtype=cache_dtype,
                                  base=w.rope_base)
    got = pool.cpu().numpy()
    # The bytes the append writes: the oracle's expected pools for two different
    # poisons agree exactly there (a written byte does not depend on the poison)
    # and differ everywhere else.
    want_5a = O.append_expected_pool(np.full(inp["n_blocks"] * bb, 0x5A, dtype=np.uint8), ckv_b, kr_b,
                                     inp["tok_seq"].numpy(), inp["tok_pos"].numpy(), inp["block_table"].numpy(),
                                     block_size=w.block_size, d_c=w.d_c, d_rope=w.d_rope, cache_dtype=cache_dtype,
                                     base=w.rope_base)
    written = want == want_5a
    # (a) no stray write: every byte outside the written rows still holds the poison, bit for bit
    stray = np.nonzero(got[~written] != 0xA5)[0]
    assert stray.size == 0, f"{stray.size} bytes outside the written rows changed"
    # (b) the set of bytes the library writes is exactly the oracle's
    written_gpu = got == pool_5a.cpu().numpy()
    assert np.array_equal(written_gpu, written), \
        f"{int((written_gpu != written).sum())} bytes differ in whether they are written"
    nb = inp["n_blocks"]
    if cache_dtype == "bf16":
        g = _bf16_pool_values(got, nb, w.block_size, w.d_c + w.d_rope)
        e = _bf16_pool_values(want, nb, w.block_size, w.d_c + w.d_rope)
        written = np.zeros((nb, w.block_size), dtype=bool)
        tbl = inp["block_table"].numpy()
        for sq, p in zip(inp["tok_seq"].numpy(), inp["tok_pos"].numpy()):
            written[tbl[sq, p // w.block_size], p % w.block_size] = True
        # one ulp of the latent; the rotated key as bounded above
        gl, el = g[written][:, :w.d_c], e[written][:, :w.d_c]
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(el), 1e-30))) - 7)
        bad = np.abs(gl - el) > ulp + ACC_ABS
        assert not bad.any(), f"latent: {int(bad.sum())} elements beyond one ulp (+{ACC_ABS})"
        _assert_rotated_close(g[written][:, w.d_c:], e[written][:, w.d_c:], "cached k_R")
    else:
        # the decoded latent: where a code differs it is one E4M3 step away (at most 1/8 relative)
        blk = 64 * w.d_c
        for b in range(nb):
            base = b * bb
            gc = O.e4m3fn_decode(got[base:base + blk])
            ec = O.e4m3fn_decode(want[base:base + blk])
            gs = got[base + blk:base + blk + 4 * 64].view(np.float32).astype(np.float64)
            es = want[base + blk:base + blk + 4 * 64].view(np.float32).astype(np.float64)
            gv = gc.reshape(64, w.d_c) * gs[:, None]
            ev = ec.reshape(64, w.d_c) * es[:, None]
            ok = np.isfinite(ev)
            assert np.all(np.abs(gv - ev)[ok] <= 0.126 * np.abs(ev)[ok] + 2.0 ** -9 * np.abs(es).max() + 1e-30)


@pytest.mark.parametrize("n_tok", [64, 37, 1, 200])
def test_absorb_from_latent_matches_oracle(n_tok, cuda_device):
    import mla_latent_kv_23_amd as M
    w = V3
    inp = S.make_inputs(w.replace(batch=1), 820, seqlens=torch.tensor([8], dtype=torch.int32))
    up = S.make_upstream_inputs(w, 821, n_tok)
    gen = torch.Generator().manual_seed(822)
    c_q = torch.randn(n_tok, up["d_cq"], generator=gen).to(torch.bfloat16)
    pos = torch.randint(0, 100000, (n_tok,), generator=gen, dtype=torch.int32)
    U.say(f"[absorb_from_latent] n_tok={n_tok}")
    d = U.dims_of(w)
    dev = cuda_device
    q_abs = M.absorb_from_latent(d, c_q.to(dev), up["w_uq"].to(dev), pos.to(dev), inp["w_uk"].to(dev))
    torch.cuda.synchronize()
    args = (c_q.double().numpy(), up["w_uq"].double().numpy(), pos.numpy(), inp["w_uk"].double().numpy(), w.d_nope,
            w.rope_base)
    want = O.query_from_latent(*args)                       # R17: q_C, q_R rounded to bf16 first
    exact = O.query_from_latent(*args, out_dtype=None)      # no intermediate rounding
    # the latent part: the bf16 bar against the exact chain, and one rounding of the R17 chain's value on
    # all but a few elements (where the float32 sum of a q_C element rounds the other way than the
    # float64 one, the 128-term absorb moves by about that element's ulp times a weight)
    U.assert_close(q_abs[..., :w.d_c], exact[..., :w.d_c], "bf16", "q_lat vs exact chain")
    g = q_abs[..., :w.d_c].double().cpu().numpy()
    e = want[..., :w.d_c]
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(e), 1e-30))) - 7)
    frac = float(np.mean(np.abs(g - e) <= 1.5 * ulp))
    assert frac >= 0.999, f"q_lat: only {frac:.5f} of the elements within 1.5 ulp of the bf16 chain"
    _assert_rotated_close(q_abs[..., w.d_c:].double().cpu().numpy(), want[..., w.d_c:], "rotated q_R")


@pytest.mark.parametrize("gated,side", [(False, False), (True, False), (True, True)])
def test_decode_step_from_hidden_states(gated, side, cuda_device):
    """DecodeStep.run_from_hidden: down-projection + append, query path + absorb, decode,
    combine and the (gated) up-projection, against the oracle's chain: the new tokens'
    latents and keys from project_down, the queries from query_from_latent.  With
    `side`, the step runs on a side stream held back by a spin kernel, so a launch
    that ignored the stream argument would run before its inputs exist."""
    import mla_latent_kv_23_amd as M
    w = V3.replace(batch=2)
    lens = [300, 70]
    inp = S.make_inputs(w, 830, seqlens=torch.tensor(lens, dtype=torch.int32))
    new_rows = S.new_token_rows(inp, 1).numpy()
    hist = np.setdiff1d(np.arange(int(sum(lens))), new_rows)
    up = S.make_upstream_inputs(w, 831, 2)
    U.say(f"[step_from_hidden] gated={gated}")
    d = U.dims_of(w)
    dev = cuda_device
    pool = U.gpu_pool(w, inp, dev, rows=hist)
    table = inp["block_table"].to(dev)
    q_pos = S.query_positions(inp["seqlens"], 1).reshape(-1)
    gate = S.make_gate_logits(w, 832, 2) if gated else None
    step = M.DecodeStep(d, 2, 1, table.shape[1], device=dev)
    args = dict(
        h=up["h"].to(dev), w_down=up["w_down"].to(dev), d_cq=up["d_cq"], w_uq=up["w_uq"].to(dev),
        q_pos=q_pos.to(dev), new_seq_id=inp["tok_seq"][new_rows].to(dev), new_pos=inp["tok_pos"][new_rows].to(dev),
        block_table=table, seqlens=inp["seqlens"].to(dev), pool=pool, w_uk=inp["w_uk"].to(dev),
        w_uv=inp["w_uv"].to(dev), gate=None if gate is None else gate.to(dev))
    if not side:
        out, _, _ = step.run_from_hidden(**args)
    else:
        if not hasattr(torch.cuda, "_sleep"):
            pytest.skip("torch.cuda._sleep is not available")
        torch.cuda.synchronize()
        stream = torch.cuda.Stream()              # default priority
        with torch.cuda.stream(stream):
            torch.cuda._sleep(20_000_000)         # a bounded spin of some milliseconds ahead of the step
            out, _, _ = step.run_from_hidden(**args, stream=stream)
        torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    cq, ckv, kr = O.project_down(up["h"].double().numpy(), up["w_down"].double().numpy(), up["d_cq"], w.d_c, w.d_rope)
    q_abs = O.query_from_latent(cq, up["w_uq"].double().numpy(), q_pos.numpy(), inp["w_uk"].double().numpy(), w.d_nope,
                                w.rope_base)
    cu = inp["cu_seqlens"].tolist()
    for b, L in enumerate(lens):
        rows = np.arange(cu[b], cu[b] + L - 1)
        c_h, kr_h = O.cached_token_values(inp["c_kv"][rows].double().numpy(), inp["k_rope"][rows].double().numpy(),
                                          np.arange(L - 1), w.cache_dtype, w.rope_base)
        c_n, kr_n = O.cached_token_values(ckv[b:b + 1], kr[b:b + 1], np.array([L - 1]), w.cache_dtype, w.rope_base)
        o_lat, _ = O.decode_absorbed_form(q_abs[b:b + 1], np.concatenate([c_h, c_n]), np.concatenate([kr_h, kr_n]),
                                          np.array([L - 1]), w.softmax_scale)
        want = O.up_proj(o_lat, inp["w_uv"].double().numpy())
        if gated:
            want = O.output_gate(want, gate[b:b + 1].double().numpy())
        U.assert_close(out[b:b + 1], want, "bf16", f"out seq {b}")
