"""GPU edge cases of the decode path whose expected values are closed forms or
properties rather than only the oracle's numbers ("Transformer升级之路：21、
MLA好在哪里？（下）", 双重投影, decoding column: the key and the value of a token
are its cached latent c, so the output is a convex combination of the c_t):

  * a zero query scores every visible token 0: the output is the plain mean of
    the visible latents and lse = ln(visible count);
  * identical latents make every convex combination equal that latent,
    whatever the weights (the rotated keys still differ by position);
  * two launches of decode + combine on the same inputs and split count give
    the same bits;
  * block-table entries outside the pool are padding: their tokens are left
    out of the softmax (never read), and a row that sees none gets 0 and -inf;
  * MLA without the decoupled RoPE part (d_rope = 0): the absorb reads no q_R
    or position, and the whole step matches the oracle's MHA form.

Every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import mla_synth as S
from oracle import mla_oracle as O
from tests import _util as U

pytestmark = pytest.mark.gpu

V3 = S.WORKLOADS["v3_bs64_ctx8k"]
# (workload, cache) cases: the tuned decode with a bf16 and an fp8 cache (32 and 128 heads), and
# the generic decode (fp32, the tiny workload's dims; bf16 with 16-token blocks)
CASES = {
    "bf16": V3.replace(batch=3, n_heads=32),
    "fp8": V3.replace(batch=3, n_heads=32, cache_dtype="fp8"),
    # 128 heads: one 128-pair work-group per query row (with an fp8 cache, the kernel that
    # reads the staged codes in place instead of expanding each tile)
    "bf16_128": V3.replace(batch=3),
    "fp8_128": V3.replace(batch=3, cache_dtype="fp8"),
    "f32_generic": S.WORKLOADS["tiny_fp32"].replace(batch=3, n_heads=4),
    "bf16_generic": V3.replace(batch=3, n_heads=16, block_size=16),
}
LENS = [300, 33, 1000]


def _decode(w, inp, q_abs_dev, dev, num_splits, table=None):
    import mla_latent_kv_23_amd as M
    d = U.dims_of(w)
    pool = U.gpu_pool(w, inp, dev, poison=0xFF)
    bt = (inp["block_table"] if table is None else table).to(dev)
    L = inp["seqlens"].to(dev)
    o_lat, lse, ws = M.decode(d, q_abs_dev, pool, bt, L, num_splits=num_splits)
    M.combine(d, L, bt.shape[1], ws, o_lat, lse, num_splits=num_splits)
    torch.cuda.synchronize()
    return o_lat, lse


def _cached(w, inp, b):
    cu = inp["cu_seqlens"].numpy()
    Lb = int(inp["seqlens"][b])
    return O.cached_token_values(inp["c_kv"][cu[b]:cu[b] + Lb].double().numpy(),
                                 inp["k_rope"][cu[b]:cu[b] + Lb].double().numpy(), np.arange(Lb), w.cache_dtype,
                                 w.rope_base)


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("num_splits", [0, 1, 5])
def test_zero_query_gives_the_mean_latent(case, num_splits, cuda_device):
    w = CASES[case]
    inp = S.make_inputs(w, 9100, seqlens=torch.tensor(LENS[:w.batch], dtype=torch.int32))
    U.say(f"[zero query] {case} splits={num_splits}")
    q = torch.zeros((w.batch, 1, w.n_heads, w.d_c + w.d_rope), dtype=S.TORCH_DTYPE[w.act_dtype], device=cuda_device)
    o_lat, lse = _decode(w, inp, q, cuda_device, num_splits)
    for b in range(w.batch):
        c, _ = _cached(w, inp, b)
        Lb = c.shape[0]
        want_o = np.broadcast_to(c.mean(axis=0), (1, w.n_heads, w.d_c))
        U.assert_close(o_lat[b], want_o, w.act_dtype, f"o_lat L={Lb}")
        got_lse = lse[b].double().cpu().numpy()
        assert np.allclose(got_lse, np.log(Lb), rtol=2e-6, atol=0), f"lse {got_lse.ravel()[:4]} vs ln {Lb}"


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("num_splits", [0, 1, 5])
def test_identical_latents_give_that_latent(case, num_splits, cuda_device):
    w = CASES[case]
    inp = S.make_inputs(w, 9200, seqlens=torch.tensor(LENS[:w.batch], dtype=torch.int32))
    cu = inp["cu_seqlens"].tolist()
    c = inp["c_kv"].clone()
    for b in range(w.batch):   # every token of sequence b caches the latent of its first token
        c[cu[b]:cu[b + 1]] = c[cu[b]]
    inp["c_kv"] = c
    U.say(f"[identical rows] {case} splits={num_splits}")
    pos = S.query_positions(inp["seqlens"], 1).numpy()
    q_abs = O.absorb_q(inp["q_nope"].double().numpy(), inp["q_rope"].double().numpy(),
                       pos[:, :, None] * np.ones((1, 1, w.n_heads), np.int64), inp["w_uk"].double().numpy(),
                       w.rope_base)
    q_dev = U.to_act(q_abs, w.act_dtype, cuda_device)
    o_lat, lse = _decode(w, inp, q_dev, cuda_device, num_splits)
    assert torch.isfinite(lse).all()
    for b in range(w.batch):
        c_b, _ = _cached(w, inp, b)
        row = c_b[0]
        if w.act_dtype == "f32":
            U.assert_close(o_lat[b], np.broadcast_to(row, (1, w.n_heads, w.d_c)), "f32", f"o_lat seq {b}")
            continue
        # bf16: the latent itself, to 1.5 units in its last place.  The weights
        # enter the matrix units rounded to bf16 (the fp8 cache's as p_t * s_t)
        # and split partials are stored in bf16, each a 2^-9 relative effect on
        # the normalised sum, below one ulp together with the final rounding.
        got = o_lat[b].double().cpu().numpy()
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(row), 1e-30))) - 7)
        ratio = np.abs(got - row[None, None, :]) / ulp[None, None, :]
        assert np.all(ratio <= 1.5), f"seq {b}: worst {float(ratio.max()):.2f} ulp"


@pytest.mark.parametrize("case", ["bf16", "fp8", "fp8_128", "bf16_generic"])
@pytest.mark.parametrize("num_splits", [0, 7])
def test_decode_and_combine_are_deterministic(case, num_splits, cuda_device):
    w = CASES[case]
    inp = S.make_inputs(w, 9300, seqlens=torch.tensor(LENS, dtype=torch.int32))
    U.say(f"[determinism] {case} splits={num_splits}")
    pos = S.query_positions(inp["seqlens"], 1).numpy()
    q_abs = O.absorb_q(inp["q_nope"].double().numpy(), inp["q_rope"].double().numpy(),
                       pos[:, :, None] * np.ones((1, 1, w.n_heads), np.int64), inp["w_uk"].double().numpy(),
                       w.rope_base)
    q_dev = U.to_act(q_abs, w.act_dtype, cuda_device)
    o1, l1 = _decode(w, inp, q_dev, cuda_device, num_splits)
    o2, l2 = _decode(w, inp, q_dev, cuda_device, num_splits)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("num_splits", [0, 1, 4])
def test_block_ids_outside_the_pool_are_padding(case, num_splits, cuda_device):
    """Entries >= the pool's block count (just past it, and far past it) inside a
    sequence's length: their tokens drop out of the softmax; a sequence whose
    only block is outside the pool gets o_lat = 0 and lse = -inf."""
    w = CASES[case]
    bs = w.block_size
    lens = [5 * bs + 17, 3 * bs, bs]
    inp = S.make_inputs(w, 9400, seqlens=torch.tensor(lens, dtype=torch.int32))
    n_blocks = inp["n_blocks"]
    table = inp["block_table"].clone()
    table[0, 2] = n_blocks + 7          # tokens 2bs .. 3bs-1 of sequence 0
    table[1, 1] = 1 << 30               # tokens bs .. 2bs-1 of sequence 1
    table[2, 0] = n_blocks              # the only block of sequence 2
    dropped = {0: range(2 * bs, 3 * bs), 1: range(bs, 2 * bs), 2: range(0, bs)}
    U.say(f"[outside pool] {case} splits={num_splits}")
    pos = S.query_positions(inp["seqlens"], 1).numpy()
    q_abs = O.absorb_q(inp["q_nope"].double().numpy(), inp["q_rope"].double().numpy(),
                       pos[:, :, None] * np.ones((1, 1, w.n_heads), np.int64), inp["w_uk"].double().numpy(),
                       w.rope_base)
    q_dev = U.to_act(q_abs, w.act_dtype, cuda_device)
    q_r = q_dev.double().cpu().numpy()
    o_lat, lse = _decode(w, inp, q_dev, cuda_device, num_splits, table=table)
    for b, Lb in enumerate(lens):
        c, kr = _cached(w, inp, b)
        keep = np.setdiff1d(np.arange(Lb), np.array(list(dropped[b])))
        if keep.size == 0:
            assert torch.all(o_lat[b] == 0)
            assert torch.all(torch.isneginf(lse[b]))
            continue
        # the remaining tokens, all visible to the query at position Lb - 1
        want_o, want_lse = O.decode_absorbed_form(q_r[b], c[keep], kr[keep], np.array([keep.size - 1]),
                                                  w.softmax_scale)
        U.assert_close(o_lat[b], want_o, w.act_dtype, f"o_lat seq {b}")
        U.assert_close(lse[b], want_lse, w.act_dtype, f"lse seq {b}")


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_step_without_rope_part(cache, cuda_device):
    """d_rope = 0: the absorb (fused with the append) gets no q_R and no
    positions, the keys are the latents alone; decode, combine and the
    up-projection against the oracle's MHA form."""
    import mla_latent_kv_23_amd as M
    w = V3.replace(batch=3, n_heads=16, d_rope=0, cache_dtype=cache)
    lens = [300, 1, 777]
    inp = S.make_inputs(w, 9500, seqlens=torch.tensor(lens, dtype=torch.int32))
    U.say(f"[no rope] {cache}")
    d = U.dims_of(w)
    dev = cuda_device
    new_rows = U.new_tokens(inp, 1)
    old = torch.ones(inp["c_kv"].shape[0], dtype=torch.bool)
    old[new_rows] = False
    pool = U.gpu_pool(w, inp, dev, poison=0xFF, rows=torch.nonzero(old)[:, 0])
    step = M.DecodeStep(d, 3, 1, inp["block_table"].shape[1], device=dev)
    import mla_latent_kv_23_amd.binding as B
    lib = B.load_library()
    # the absorb alone, with null q_R and positions, through the C ABI
    q_abs = torch.empty((3, w.n_heads, w.d_c), dtype=torch.bfloat16, device=dev)
    qn = inp["q_nope"].reshape(3, w.n_heads, -1).to(dev)
    import ctypes
    st = lib.mla_absorb_q(ctypes.byref(d), 3, qn.data_ptr(), None, None, inp["w_uk"].to(dev).data_ptr(),
                          q_abs.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    want_q = O.absorb_q(inp["q_nope"].reshape(3, w.n_heads, -1).double().numpy(),
                        np.zeros((3, w.n_heads, 0)), np.zeros((3, 1), np.int64), inp["w_uk"].double().numpy(),
                        w.rope_base)
    torch.cuda.synchronize()
    U.assert_close_ulp(q_abs, want_q, "bf16", "q_abs without RoPE")
    out, o_lat, lse = step.run(
        q_nope=qn, q_rope=inp["q_rope"].reshape(3, w.n_heads, 0).to(dev),
        q_pos=U.q_positions_flat(inp, 1).to(dev),
        new_c_kv=inp["c_kv"][new_rows].to(dev), new_k_rope=inp["k_rope"][new_rows].to(dev),
        new_seq_id=inp["tok_seq"][new_rows].to(dev), new_pos=inp["tok_pos"][new_rows].to(dev),
        block_table=inp["block_table"].to(dev), seqlens=inp["seqlens"].to(dev), pool=pool,
        w_uk=inp["w_uk"].to(dev), w_uv=inp["w_uv"].to(dev))
    torch.cuda.synchronize()
    ref = O.decode_batch(inp, q_per_seq=1, scale=w.softmax_scale, base=w.rope_base, cache_dtype=cache)
    U.assert_close(out.view(3, 1, w.n_heads, w.d_v), ref["o"], "bf16", "o")
    U.assert_close(o_lat, ref["o_lat"], "bf16", "o_lat")
    U.assert_close(lse, ref["lse"], "bf16", "lse")
