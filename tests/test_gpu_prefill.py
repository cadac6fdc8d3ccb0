"""GPU parity of the MHA-form prefill (mla_prefill, mla_prefill_paged) against
the CPU oracle's exact MHA form (float64 throughout: no operand is rounded), on
packed sequences whose lengths cover one token, partial and several 64-key
blocks and 128-query blocks, with 16 and 128 heads, a 4096-token prompt, and
bf16 and fp8 paged caches.  The library rotates the RoPE parts by the absorb's
rule and runs the contractions on bf16 matrix units with fp32 sums; the bar is
the bf16 one.  All calls go through the C ABI."""
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
                                              w.softmax_scale, w.rope_base)
        U.assert_close(out[sl], want_o, "bf16", f"out seq {b} L={L}")
        U.assert_close(lse[sl], want_lse, "bf16", f"lse seq {b} L={L}")


def test_prefill_long_prompt_sampled_heads(cuda_device):
    """One 4096-token prompt and a short one, all 128 heads computed, checked
    against the exact MHA form on sampled heads (every query row)."""
    import mla_latent_kv_23_amd as M
    w = V3
    lens = [4096, 77]
    heads_chk = [0, 41, 127]
    inp = S.make_prefill_inputs(w, 4096, torch.tensor(lens, dtype=torch.int32))
    U.say(f"[prefill long] lens={lens} heads={heads_chk}")
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
                                              w.softmax_scale, w.rope_base, heads=heads_chk)
        U.assert_close(out[sl][:, heads_chk], want_o, "bf16", f"out seq {b} L={L}")
        U.assert_close(lse[sl][:, heads_chk], want_lse, "bf16", f"lse seq {b} L={L}")


def test_prefill_reuses_one_workspace(cuda_device):
    """Two prefills in a row on one workspace (sized for the larger), the second
    with fewer and shorter prompts: the decompressed keys and values, the
    rotation table and the rotated k_R of the first call may not leak into it."""
    import mla_latent_kv_23_amd as M
    w = V3.replace(n_heads=16)
    dev = cuda_device
    ws = None
    for seed, lens in ((7001, [300, 129]), (7002, [65])):
        inp = S.make_prefill_inputs(w, seed, torch.tensor(lens, dtype=torch.int32))
        U.say(f"[prefill reuse] lens={lens}")
        d = U.dims_of(w)
        out, lse, ws = M.prefill(d, inp["q_nope"].to(dev), inp["q_rope"].to(dev), inp["c_kv"].to(dev),
                                 inp["k_rope"].to(dev), inp["cu_seqlens"].to(dev), max(lens), inp["w_uk"].to(dev),
                                 inp["w_uv"].to(dev), workspace=ws)
        torch.cuda.synchronize()
        cu = inp["cu_seqlens"].tolist()
        for b, L in enumerate(lens):
            sl = slice(cu[b], cu[b] + L)
            want_o, want_lse = O.prefill_mha_form(inp["q_nope"][sl].double().numpy(),
                                                  inp["q_rope"][sl].double().numpy(),
                                                  inp["c_kv"][sl].double().numpy(), inp["k_rope"][sl].double().numpy(),
                                                  inp["w_uk"].double().numpy(), inp["w_uv"].double().numpy(),
                                                  w.softmax_scale, w.rope_base)
            U.assert_close(out[sl], want_o, "bf16", f"out seq {b} L={L}")
            U.assert_close(lse[sl], want_lse, "bf16", f"lse seq {b} L={L}")


def test_prefill_paged_runs_on_the_callers_stream(cuda_device):
    """Chunked prefill (gather, rotation, decompression, attention) on a side
    stream held back by a spin kernel: every launch must follow the stream."""
    import mla_latent_kv_23_amd as M
    if not hasattr(torch.cuda, "_sleep"):
        pytest.skip("torch.cuda._sleep is not available")
    lens, qlens = [700, 200], [200, 33]
    w = V3.replace(n_heads=16)
    inp = S.make_chunk_prefill_inputs(w, 7300, torch.tensor(lens, dtype=torch.int32),
                                      torch.tensor(qlens, dtype=torch.int32))
    U.say("[prefill_paged stream]")
    d = U.dims_of(w)
    dev = cuda_device
    pool = U.gpu_pool(w, inp, dev)
    args = [inp["q_nope"].to(dev), inp["q_rope"].to(dev), inp["cu_q"].to(dev), max(qlens), inp["cu_k"].to(dev),
            sum(lens), pool, inp["block_table"].to(dev), inp["w_uk"].to(dev), inp["w_uv"].to(dev)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()                    # default priority
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)             # a bounded spin of some milliseconds ahead of the call
        out, lse, _ = M.prefill_paged(d, *args, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    cu_q, cu_k = inp["cu_q"].tolist(), inp["cu_k"].tolist()
    for b, (L, Lq) in enumerate(zip(lens, qlens)):
        ks, qs = slice(cu_k[b], cu_k[b] + L), slice(cu_q[b], cu_q[b] + Lq)
        c, kr = O.cached_token_values(inp["c_kv"][ks].double().numpy(), inp["k_rope"][ks].double().numpy(),
                                      np.arange(L), w.cache_dtype, w.rope_base)
        want_o, want_lse = O.prefill_chunk_mha_form(inp["q_nope"][qs].double().numpy(),
                                                    inp["q_rope"][qs].double().numpy(), c, kr,
                                                    inp["w_uk"].double().numpy(), inp["w_uv"].double().numpy(),
                                                    w.softmax_scale, w.rope_base, heads=list(range(16)))
        U.assert_close(out[qs], want_o, "bf16", f"out seq {b} L={L} Lq={Lq}")
        U.assert_close(lse[qs], want_lse, "bf16", f"lse seq {b} L={L} Lq={Lq}")


def test_prefill_rejects_unsupported_dims(cuda_device):
    import mla_latent_kv_23_amd as M
    w = S.WORKLOADS["tiny_fp32"]
    d = U.dims_of(w)
    assert M.prefill_workspace_bytes(d, 10) == 0


@pytest.mark.parametrize("heads,lens,qlens,cache", [
    (16, [1000, 129, 64, 300], [70, 1, 64, 300], "bf16"),    # prefix + chunk, one query, one block, whole prompt
    (128, [700, 200], [200, 33], "bf16"),
    (16, [5000, 77], [129, 0], "bf16"),                       # a sequence with no queries
    (16, [1000, 129, 64], [70, 1, 64], "fp8"),
    (128, [700, 200], [200, 33], "fp8"),
])
def test_prefill_paged_matches_oracle(heads, lens, qlens, cache, cuda_device):
    """Chunked prefill: each sequence's newest tokens (already in the paged cache,
    written by the library's append) attend to the whole cached prompt.  With an
    fp8 cache the latent enters as bf16(code * scale) on both sides."""
    import mla_latent_kv_23_amd as M
    w = V3.replace(n_heads=heads, cache_dtype=cache)
    inp = S.make_chunk_prefill_inputs(w, 600 + heads + len(lens), torch.tensor(lens, dtype=torch.int32),
                                      torch.tensor(qlens, dtype=torch.int32))
    U.say(f"[prefill_paged] H={heads} lens={lens} qlens={qlens} cache={cache}")
    d = U.dims_of(w)
    dev = cuda_device
    pool = U.gpu_pool(w, inp, dev)
    out, lse, _ = M.prefill_paged(d, inp["q_nope"].to(dev), inp["q_rope"].to(dev), inp["cu_q"].to(dev), max(qlens),
                                  inp["cu_k"].to(dev), sum(lens), pool, inp["block_table"].to(dev),
                                  inp["w_uk"].to(dev), inp["w_uv"].to(dev))
    torch.cuda.synchronize()
    heads_chk = list(range(heads)) if heads <= 16 else [0, 5, 64, 127]
    cu_q, cu_k = inp["cu_q"].tolist(), inp["cu_k"].tolist()
    for b, (L, Lq) in enumerate(zip(lens, qlens)):
        if Lq == 0:
            continue
        ks, qs = slice(cu_k[b], cu_k[b] + L), slice(cu_q[b], cu_q[b] + Lq)
        c, kr = O.cached_token_values(inp["c_kv"][ks].double().numpy(), inp["k_rope"][ks].double().numpy(),
                                      np.arange(L), w.cache_dtype, w.rope_base)
        want_o, want_lse = O.prefill_chunk_mha_form(inp["q_nope"][qs].double().numpy(),
                                                    inp["q_rope"][qs].double().numpy(), c, kr,
                                                    inp["w_uk"].double().numpy(), inp["w_uv"].double().numpy(),
                                                    w.softmax_scale, w.rope_base, heads=heads_chk)
        U.assert_close(out[qs][:, heads_chk], want_o, "bf16", f"out seq {b} L={L} Lq={Lq}")
        U.assert_close(lse[qs][:, heads_chk], want_lse, "bf16", f"lse seq {b} L={L} Lq={Lq}")


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
@pytest.mark.parametrize("block_size", [16, 32, 128])
def test_prefill_paged_block_sizes(block_size, cache, cuda_device):
    """Chunked prefill reading the paged cache through blocks of 16, 32 and 128
    tokens (a shuffled table with padded entries) in both cache formats."""
    import mla_latent_kv_23_amd as M
    lens, qlens = [300, 77], [100, 77]
    w = V3.replace(n_heads=16, cache_dtype=cache, block_size=block_size)
    inp = S.make_chunk_prefill_inputs(w, 6100 + block_size, torch.tensor(lens, dtype=torch.int32),
                                      torch.tensor(qlens, dtype=torch.int32))
    U.say(f"[prefill_paged blocks] block_size={block_size} cache={cache}")
    d = U.dims_of(w)
    dev = cuda_device
    pool = U.gpu_pool(w, inp, dev)
    out, lse, _ = M.prefill_paged(d, inp["q_nope"].to(dev), inp["q_rope"].to(dev), inp["cu_q"].to(dev), max(qlens),
                                  inp["cu_k"].to(dev), sum(lens), pool, inp["block_table"].to(dev),
                                  inp["w_uk"].to(dev), inp["w_uv"].to(dev))
    torch.cuda.synchronize()
    cu_q, cu_k = inp["cu_q"].tolist(), inp["cu_k"].tolist()
    for b, (L, Lq) in enumerate(zip(lens, qlens)):
        ks, qs = slice(cu_k[b], cu_k[b] + L), slice(cu_q[b], cu_q[b] + Lq)
        c, kr = O.cached_token_values(inp["c_kv"][ks].double().numpy(), inp["k_rope"][ks].double().numpy(),
                                      np.arange(L), w.cache_dtype, w.rope_base)
        want_o, want_lse = O.prefill_chunk_mha_form(inp["q_nope"][qs].double().numpy(),
                                                    inp["q_rope"][qs].double().numpy(), c, kr,
                                                    inp["w_uk"].double().numpy(), inp["w_uv"].double().numpy(),
                                                    w.softmax_scale, w.rope_base, heads=list(range(16)))
        U.assert_close(out[qs], want_o, "bf16", f"out seq {b} L={L} Lq={Lq}")
        U.assert_close(lse[qs], want_lse, "bf16", f"lse seq {b} L={L} Lq={Lq}")


@pytest.mark.parametrize("paged", [False, True])
def test_prefill_output_gate(paged, cuda_device):
    """Gated MLA in prefill: out = sigmoid(gate) * o against the oracle's gated
    prefill; lse is the ungated one."""
    import mla_latent_kv_23_amd as M
    w = V3.replace(n_heads=16)
    lens, qlens, dev = [300, 45], [100, 45], cuda_device
    d = U.dims_of(w)
    U.say(f"[prefill_gate] paged={paged}")
    if paged:
        inp = S.make_chunk_prefill_inputs(w, 700, torch.tensor(lens, dtype=torch.int32),
                                          torch.tensor(qlens, dtype=torch.int32))
        pool = U.gpu_pool(w, inp, dev)
        gate = S.make_gate_logits(w, 701, sum(qlens))
        out, lse, _ = M.prefill_paged(d, inp["q_nope"].to(dev), inp["q_rope"].to(dev), inp["cu_q"].to(dev),
                                      max(qlens), inp["cu_k"].to(dev), sum(lens), pool, inp["block_table"].to(dev),
                                      inp["w_uk"].to(dev), inp["w_uv"].to(dev), gate=gate.to(dev))
        cu_q, cu_k = inp["cu_q"].tolist(), inp["cu_k"].tolist()
    else:
        inp = S.make_prefill_inputs(w, 702, torch.tensor(lens, dtype=torch.int32))
        gate = S.make_gate_logits(w, 703, sum(lens))
        out, lse, _ = M.prefill(d, inp["q_nope"].to(dev), inp["q_rope"].to(dev), inp["c_kv"].to(dev),
                                inp["k_rope"].to(dev), inp["cu_seqlens"].to(dev), max(lens), inp["w_uk"].to(dev),
                                inp["w_uv"].to(dev), gate=gate.to(dev))
        cu_q = cu_k = inp["cu_seqlens"].tolist()
        qlens = lens
    torch.cuda.synchronize()
    wk, wv = inp["w_uk"].double().numpy(), inp["w_uv"].double().numpy()
    for b, (L, Lq) in enumerate(zip(lens, qlens)):
        ks, qs = slice(cu_k[b], cu_k[b] + L), slice(cu_q[b], cu_q[b] + Lq)
        qn, qr = inp["q_nope"][qs].double().numpy(), inp["q_rope"][qs].double().numpy()
        if paged:
            c, kr = O.cached_token_values(inp["c_kv"][ks].double().numpy(), inp["k_rope"][ks].double().numpy(),
                                          np.arange(L), w.cache_dtype, w.rope_base)
            o, l = O.prefill_chunk_mha_form(qn, qr, c, kr, wk, wv, w.softmax_scale, w.rope_base)
        else:
            o, l = O.prefill_mha_form(qn, qr, inp["c_kv"][ks].double().numpy(), inp["k_rope"][ks].double().numpy(),
                                      wk, wv, w.softmax_scale, w.rope_base)
        want = O.output_gate(o, gate[qs].double().numpy())
        U.assert_close(out[qs], want, "bf16", f"gated out seq {b}")
        U.assert_close(lse[qs], l, "bf16", f"lse seq {b}")
