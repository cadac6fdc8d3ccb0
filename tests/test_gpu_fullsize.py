"""Full-size parity: each workload at its real size, run end to end on the GPU
(absorb -> append of the whole history -> decode -> combine -> up-projection,
the launch configuration the benchmark times), checked against the CPU oracle
on sampled sequences and heads (the oracle computes them one by one).  The
samples include the shortest and longest sequence of the ragged workload."""
import numpy as np
import pytest
import torch

import mla_synth as S
from oracle import mla_oracle as O
from tests import _util as U

pytestmark = pytest.mark.gpu

SAMPLES = {   # workload -> (sequences, heads); None = all
    "tiny_fp32": (None, None),
    "mid_bf16": ([0, 9, 15], None),
    "v3_bs64_ctx8k": ([0, 37, 63], [0, 77, 127]),
    "ragged_sq2": ("extremes", [0, 64, 127]),
    "fp8_ctx64k": ([0, 31], [5, 100]),
}


def run_chain(w, inp, dev, num_splits=0):
    import mla_latent_kv_23_amd as M
    d = U.dims_of(w)
    B, sq = inp["q_nope"].shape[:2]
    n_tok = B * sq
    pool = U.gpu_pool(w, inp, dev, poison=0xFF)            # whole cache (the new tokens included)
    step = M.DecodeStep(d, B, sq, inp["block_table"].shape[1], num_splits=num_splits, device=dev)
    out, o_lat, lse = step.run(
        q_nope=inp["q_nope"].reshape(n_tok, w.n_heads, -1).to(dev),
        q_rope=inp["q_rope"].reshape(n_tok, w.n_heads, -1).to(dev),
        q_pos=U.q_positions_flat(inp, sq).to(dev), new_c_kv=None, new_k_rope=None, new_seq_id=None,
        new_pos=None, block_table=inp["block_table"].to(dev), seqlens=inp["seqlens"].to(dev), pool=pool,
        w_uk=inp["w_uk"].to(dev), w_uv=inp["w_uv"].to(dev))
    torch.cuda.synchronize()
    return out.view(B, sq, w.n_heads, w.d_v).cpu(), o_lat.cpu(), lse.cpu()


@pytest.mark.parametrize("name", S.WORKLOAD_ORDER)
def test_full_size_sampled(name, cuda_device):
    w = S.WORKLOADS[name]
    U.say(f"[full] {name}: generating inputs")
    inp = S.make_inputs(w, S.SEEDS[name])
    U.say(f"[full] {name}: GPU chain, {int(inp['seqlens'].sum())} cached tokens")
    out, o_lat, lse = run_chain(w, inp, cuda_device)
    seqs, heads = SAMPLES[name]
    if seqs == "extremes":
        L = inp["seqlens"]
        seqs = sorted({int(torch.argmin(L)), int(torch.argmax(L)), 7})
    U.say(f"[full] {name}: oracle on sequences {seqs}, heads {heads}")
    ref = O.decode_batch(inp, q_per_seq=w.q_per_seq, scale=w.softmax_scale, base=w.rope_base,
                         cache_dtype=w.cache_dtype, seqs=seqs, heads=heads)
    sel_s = list(range(w.batch)) if seqs is None else seqs
    sel_h = list(range(w.n_heads)) if heads is None else heads
    got_o = out[sel_s][:, :, sel_h]
    got_ol = o_lat[sel_s][:, :, sel_h]
    got_lse = lse[sel_s][:, :, sel_h]
    U.assert_close(got_o, ref["o"], w.act_dtype, f"{name} o")
    U.assert_close(got_ol, ref["o_lat"], w.act_dtype, f"{name} o_lat")
    U.assert_close(got_lse, ref["lse"], w.act_dtype, f"{name} lse")
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


def test_split_counts_agree_at_full_size(cuda_device):
    """The V3-shape workload with one work unit per sequence piece count 1, the
    default, and more units than CUs: all within rounding of each other and of
    the oracle on one sampled sequence."""
    w = S.WORKLOADS["v3_bs64_ctx8k"].replace(batch=8)
    inp = S.make_inputs(w, S.SEEDS["v3_bs64_ctx8k"] + 17)
    ref = O.decode_batch(inp, q_per_seq=1, scale=w.softmax_scale, base=w.rope_base, cache_dtype="bf16",
                         seqs=[3], heads=[0, 64, 127])
    for ns in [1, 0, 8, 1000]:
        U.say(f"[splits] num_splits={ns}")
        out, o_lat, lse = run_chain(w, inp, cuda_device, num_splits=ns)
        U.assert_close(out[[3]][:, :, [0, 64, 127]], ref["o"], "bf16", f"o splits={ns}")
        U.assert_close(lse[[3]][:, :, [0, 64, 127]], ref["lse"], "bf16", f"lse splits={ns}")
