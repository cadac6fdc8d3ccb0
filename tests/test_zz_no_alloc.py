"""mla_decode_noalloc (decode + split merge with the partials in the library's
static device array) against mla_decode + mla_combine on a caller workspace:
two calls in a row through the C ABI, the second on a smaller problem, each
bit-identical to the workspace path (the same kernels, another buffer), and
both within the bf16 bar of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import mla_synth as S
from oracle import mla_oracle as O
from tests import _util as U

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_noalloc_decode_equals_the_workspace_path(cache, cuda_device):
    import mla_latent_kv_23_amd as M
    from mla_latent_kv_23_amd import binding as B
    lib = B.load_library()
    dev = cuda_device
    for seed, batch, heads, lens, splits in ((9700, 3, 128, [900, 257, 1500], 0), (9701, 2, 64, [33, 200], 7)):
        w = S.WORKLOADS["v3_bs64_ctx8k"].replace(batch=batch, n_heads=heads, cache_dtype=cache)
        inp = S.make_inputs(w, seed, seqlens=torch.tensor(lens, dtype=torch.int32))
        U.say(f"[noalloc] {cache} H={heads} lens={lens} splits={splits}")
        d = U.dims_of(w)
        pos = S.query_positions(inp["seqlens"], 1).numpy()
        q_abs = O.absorb_q(inp["q_nope"].double().numpy(), inp["q_rope"].double().numpy(),
                           pos[:, :, None] * np.ones((1, 1, heads), np.int64), inp["w_uk"].double().numpy(),
                           w.rope_base)
        q_dev = U.to_act(q_abs, "bf16", dev)
        pool = U.gpu_pool(w, inp, dev, poison=0xFF)
        bt, L = inp["block_table"].to(dev), inp["seqlens"].to(dev)
        # the workspace path
        o_ref, l_ref, ws = M.decode(d, q_dev, pool, bt, L, num_splits=splits)
        M.combine(d, L, bt.shape[1], ws, o_ref, l_ref, num_splits=splits)
        # the no-allocation path (outputs poisoned first)
        o = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(l_ref, float("nan"))
        n_pool = pool.numel() // M.cache_block_bytes(d)
        st = lib.mla_decode_noalloc(ctypes.byref(d), batch, 1, q_dev.data_ptr(), pool.data_ptr(), n_pool,
                                    bt.data_ptr(), bt.shape[1], L.data_ptr(), splits, o.data_ptr(), lse.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
        assert st == 0, st
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32))
        q_r = q_dev.double().cpu().numpy()
        cu = inp["cu_seqlens"].numpy()
        for b, Lb in enumerate(lens):
            c, kr = O.cached_token_values(inp["c_kv"][cu[b]:cu[b] + Lb].double().numpy(),
                                          inp["k_rope"][cu[b]:cu[b] + Lb].double().numpy(), np.arange(Lb), cache,
                                          w.rope_base)
            want_o, want_lse = O.decode_absorbed_form(q_r[b], c, kr, pos[b], w.softmax_scale)
            U.assert_close(o[b], want_o, "bf16", f"o_lat seq {b}")
            U.assert_close(lse[b], want_lse, "bf16", f"lse seq {b}")
