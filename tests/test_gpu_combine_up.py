"""mla_combine_up_proj (the split merge fused with the up-projection) against
mla_combine + mla_up_proj(_gated) on the same decode: out and lse bit for bit,
and out against the oracle's up-projection of the exact attention output.
Cases: split and unsplit sequences in one batch (the fused kernel copies the
rows the decode finished itself), a one-token sequence, forced split counts,
two query rows, 16 heads, the fp8 cache, the output gate, and a batch that is
not a multiple of the 32-token work-group."""
import numpy as np
import pytest
import torch

import mla_synth as S
from oracle import mla_oracle as O
from tests import _util as U

pytestmark = pytest.mark.gpu

CASES = [
    # (id, heads, q_per_seq, lens, splits, cache, gated)
    ("v3-mixed", 128, 1, [900, 40, 1500, 1, 257, 3000], 0, "bf16", False),
    ("v3-gate", 128, 1, [700, 2100, 65, 1200], 0, "bf16", True),
    ("v3-splits7", 128, 1, [33, 200, 999], 7, "bf16", False),
    ("v3-one-split", 128, 1, [500, 1300], 1, "bf16", False),
    ("rows2", 128, 2, [600, 1800, 75], 0, "bf16", True),
    ("h16", 16, 1, [4000, 17, 2500, 800, 1], 0, "bf16", False),
    ("fp8", 128, 1, [1000, 64, 2200], 0, "fp8", False),
    ("t37", 128, 1, [300 + 37 * i for i in range(37)], 0, "bf16", False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_combine_up_proj_equals_the_two_calls(case, cuda_device):
    import mla_latent_kv_23_amd as M
    name, heads, sq, lens, splits, cache, gated = case
    dev = cuda_device
    batch = len(lens)
    w = S.WORKLOADS["v3_bs64_ctx8k"].replace(batch=batch, n_heads=heads, q_per_seq=sq, cache_dtype=cache)
    inp = S.make_inputs(w, 9800 + len(name), seqlens=torch.tensor(lens, dtype=torch.int32))
    U.say(f"[combine_up] {name}: H={heads} rows={sq} lens={lens} splits={splits} cache={cache} gate={gated}")
    d = U.dims_of(w)
    n_tok = batch * sq
    pos = S.query_positions(inp["seqlens"], sq).numpy()
    q_abs = O.absorb_q(inp["q_nope"].double().numpy(), inp["q_rope"].double().numpy(),
                       pos[:, :, None] * np.ones((1, 1, heads), np.int64), inp["w_uk"].double().numpy(), w.rope_base)
    q_dev = U.to_act(q_abs, "bf16", dev)
    pool = U.gpu_pool(w, inp, dev, poison=0xFF)
    bt, L = inp["block_table"].to(dev), inp["seqlens"].to(dev)
    w_uv = inp["w_uv"].to(dev)
    gate = S.make_gate_logits(w, 9900, n_tok).to(dev) if gated else None

    # decode into poisoned outputs: rows it does not finish itself keep the poison
    # (o_lat a finite 7.0, so a fused kernel that read such a row would differ)
    o_pre = torch.full((batch, sq, heads, d.d_c), 7.0, dtype=torch.bfloat16, device=dev)
    lse_pre = torch.full((batch, sq, heads), float("nan"), dtype=torch.float32, device=dev)
    o_lat, lse, ws = M.decode(d, q_dev, pool, bt, L, num_splits=splits, o_latent=o_pre, lse=lse_pre)
    torch.cuda.synchronize()
    o_dec, lse_dec = o_lat.clone(), lse.clone()          # as the decode left them
    # the two calls
    M.combine(d, L, bt.shape[1], ws, o_lat, lse, num_splits=splits)
    out_ref = M.up_proj(d, o_lat.view(n_tok, heads, -1), w_uv, gate=gate)
    # the fused call, on the decode's own outputs, without and with the merged rows written back
    for write_latent in (False, True):
        o2, lse2 = o_dec.clone(), lse_dec.clone()
        out = torch.full((n_tok, heads, d.d_v), float("nan"), dtype=torch.bfloat16, device=dev)
        M.combine_up_proj(d, L, bt.shape[1], ws, o2, lse2, w_uv, out=out, num_splits=splits, gate=gate,
                          write_latent=write_latent)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16)), "out differs from combine + up_proj"
        assert torch.equal(lse2.view(torch.int32), lse.view(torch.int32)), "lse differs from combine"
        want_lat = o_lat if write_latent else o_dec          # merged rows, or the rows as decode left them
        assert torch.equal(o2.view(torch.int16), want_lat.view(torch.int16)), f"o_latent (write_latent={write_latent})"

    # against the oracle: the exact attention output, projected in float64
    q_r = q_dev.double().cpu().numpy()
    cu = inp["cu_seqlens"].numpy()
    w_uv_r = inp["w_uv"].double().numpy()
    g_r = gate.double().cpu().numpy().reshape(batch, sq, heads, -1) if gated else None
    got = out.double().cpu().numpy().reshape(batch, sq, heads, -1)
    for b, Lb in enumerate(lens):
        c, kr = O.cached_token_values(inp["c_kv"][cu[b]:cu[b] + Lb].double().numpy(),
                                      inp["k_rope"][cu[b]:cu[b] + Lb].double().numpy(), np.arange(Lb), cache,
                                      w.rope_base)
        want_lat, _ = O.decode_absorbed_form(q_r[b], c, kr, pos[b], w.softmax_scale)
        want = O.up_proj(want_lat, w_uv_r)
        if gated:
            want = O.output_gate(want, g_r[b])
        U.assert_close(torch.from_numpy(got[b]).to(torch.bfloat16), want, "bf16", f"out seq {b} L={Lb}")


def test_decode_step_without_the_latent(cuda_device):
    """DecodeStep(keep_latent=False) runs the merge and the up-projection as one
    call and returns the same out and lse as the step that keeps the latent."""
    import mla_latent_kv_23_amd as M
    dev = cuda_device
    lens = [1200, 90, 2600, 500] + [150 + 41 * i for i in range(60)]   # 64 rows: the step fuses the merge
    w = S.WORKLOADS["v3_bs64_ctx8k"].replace(batch=len(lens))
    inp = S.make_inputs(w, 9950, seqlens=torch.tensor(lens, dtype=torch.int32))
    d = U.dims_of(w)
    B, sq, H = len(lens), 1, w.n_heads
    n_tok = B * sq
    rows = S.new_token_rows(inp, sq)
    hist = torch.ones(inp["c_kv"].shape[0], dtype=torch.bool)
    hist[rows] = False
    hist_rows = torch.nonzero(hist)[:, 0]
    outs = []
    for keep in (True, False):
        pool = torch.full((inp["n_blocks"] * M.cache_block_bytes(d),), 0xFF, dtype=torch.uint8, device=dev)
        bt = inp["block_table"].to(dev)
        M.append_cache(d, inp["c_kv"][hist_rows].to(dev), inp["k_rope"][hist_rows].to(dev),
                       inp["tok_seq"][hist_rows].to(dev), inp["tok_pos"][hist_rows].to(dev), bt, pool)
        step = M.DecodeStep(d, B, sq, bt.shape[1], device=dev, keep_latent=keep)
        out, o_lat, lse = step.run(
            q_nope=inp["q_nope"].reshape(n_tok, H, -1).to(dev), q_rope=inp["q_rope"].reshape(n_tok, H, -1).to(dev),
            q_pos=S.query_positions(inp["seqlens"], sq).reshape(-1).to(dev),
            new_c_kv=inp["c_kv"][rows].to(dev), new_k_rope=inp["k_rope"][rows].to(dev),
            new_seq_id=inp["tok_seq"][rows].to(dev), new_pos=inp["tok_pos"][rows].to(dev), block_table=bt,
            seqlens=inp["seqlens"].to(dev), pool=pool, w_uk=inp["w_uk"].to(dev), w_uv=inp["w_uv"].to(dev))
        torch.cuda.synchronize()
        assert step.fuse_merge
        assert (o_lat is None) == (not keep)
        outs.append((out.clone(), lse.clone()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))
