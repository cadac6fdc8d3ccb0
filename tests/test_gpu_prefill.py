"""GPU parity of the MHA-form prefill (mla_prefill) against the CPU oracle, on
packed sequences whose lengths cover one token, partial and several 64-key
blocks and 128-query blocks, with 16 and 128 heads.  The oracle rounds the
rotated query part and the decompressed keys and values to bf16, where the
library's matrix-unit operands are rounded (mla.h states these points); the
rest is float64.  All calls go through the C ABI."""
import numpy as np
import pytest
import torch

import mla_synth as S
from oracle import mla_oracle as O
from tests import _util as U

pytestmark = pytest.mark.gpu

V3 = S.WORKLOADS["v3_bs64_ctx8k"]


@pytest.mark.parametrize("heads,lens", [(16, [1, 70, 300]), (128, [129, 64, 5]), (16, [512, 33])])
def test_prefill_matches_oracle(heads, lens, cuda_device):
    import mla_latent_kv_23_amd as M
    w = V3.replace(n_heads=heads)
    inp = S.make_prefill_inputs(w, 500 + heads + len(lens), torch.tensor(lens, dtype=torch.int32))
    U.say(f"[prefill] H={heads} lens={lens}")
    d = U.dims_of(w)
    dev = cuda_device
    out, lse, _ = M.prefill(d, inp["q_nope"].to(dev), inp["q_rope"].to(dev), inp["c_kv"].to(dev),
                            inp["k_rope"].to(dev), inp["cu_seqlens"].to(dev), max(lens), inp["w_uk"].to(dev),
                            inp["w_uv"].to(dev))
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"].tolist()
    for b, L in enumerate(lens):
        sl = slice(cu[b], cu[b] + L)
        want_o, want_lse = O.prefill_mha_form(inp["q_nope"][sl].double().numpy(), inp["q_rope"][sl].double().numpy(),
                                              inp["c_kv"][sl].double().numpy(), inp["k_rope"][sl].double().numpy(),
                                              inp["w_uk"].double().numpy(), inp["w_uv"].double().numpy(),
                                              w.softmax_scale, w.rope_base, operand_dtype="bf16")
        U.assert_close(out[sl], want_o, "bf16", f"out seq {b} L={L}")
        U.assert_close(lse[sl], want_lse, "bf16", f"lse seq {b} L={L}")


def test_prefill_rejects_unsupported_dims(cuda_device):
    import mla_latent_kv_23_amd as M
    w = S.WORKLOADS["tiny_fp32"]
    d = U.dims_of(w)
    assert M.prefill_workspace_bytes(d, 10) == 0
