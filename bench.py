"""Benchmark: one MLA decode step (absorb -> append -> decode -> combine ->
up-projection) per layer on one MI355X, on the DeepSeek-V3-shape workload
(64 sequences x 8192 cached tokens, 128 heads, 512-wide latent + 64-wide RoPE
key, bf16, 64-token paged blocks with a shuffled block table).

Prints one JSON line.  `value` is whole-step throughput (query tokens per
second) with every input resident in HBM.  `roofline` reports the decode
kernel (the dominant one) against the HBM bound: algorithmic bytes = the
cache read once (1152 B per cached token), divided by the decode launch time
measured with HIP events around each decode launch inside the timed region
(events created without the system-scope fence, so that recording them does
not write back and invalidate the caches between kernels).
`cpu_baseline` times the CPU oracle (non-absorbed form, float64) on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0         # MI355X dense bf16 MFMA

# HBM traffic of the decode kernel measured with rocprofv3 counters (FETCH_SIZE,
# WRITE_SIZE, each scaled by its reading for a plain copy of known size); the
# summary records a hash of the kernel sources it was measured on, and the
# figure is reported only while the sources still match.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode576_v3_bs64_ctx8k_traffic.md")
# the device code of the decode kernel (its file, its tile helpers, the shared device helpers)
KERNEL_SOURCES = ["decode_latent576.hip", "decode_tile.h", "mla_device.h"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mla_latent_kv_23_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """Bytes per decode launch from the committed counter summary, or None when
    the summary is missing or was taken on other kernel sources."""
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    vals = {}
    with open(TRAFFIC_PROFILE) as f:
        for line in f:
            if ":" in line and line.strip().startswith(("traffic_bytes_per_launch", "kernel_sources_sha256")):
                k, v = line.strip().split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_sources_sha256") != kernel_source_hash():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the chip needs tens of ms of work to reach its steady clocks: with 5 warm-up steps the
    # first timed steps run ~10% slower than the steady state a serving loop sees
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="v3_bs64_ctx8k")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--cpu-sample-seqs", type=int, default=16,
                    help="sequences of the workload the CPU oracle is timed on (0 = skip)")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode+combine calls (for profiling)")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="touch a scratch buffer of this many MiB before every step (outside the kernels' events) so "
                         "that a cache smaller than the 256 MB MALL is read from HBM; the step time is then the sum "
                         "of per-step event brackets instead of the outer bracket")
    ap.add_argument("--flush-mode", choices=("read", "write"), default="read",
                    help="how the scratch buffer evicts the cache: read it (clean lines, like the other layers' "
                         "cache reads between two steps of one layer) or overwrite it (dirty lines, whose "
                         "write-back then competes with the next step's reads)")
    ap.add_argument("--upstream", action="store_true",
                    help="start the step from the hidden state: mla_project_down (W_DQ, W_DKV, W_KR and the append) "
                         "and mla_absorb_from_latent (W_UQ and the absorb) replace the append and the absorb")
    ap.add_argument("--separate-merge", action="store_true",
                    help="merge the key splits and up-project with two calls (mla_combine, mla_up_proj) also where "
                         "the step would use the one fused call (mla_combine_up_proj: when one work-group per head "
                         "and 32 query rows fills the chip)")
    ap.add_argument("--gated", action="store_true",
                    help="gated MLA: the up-projection applies a sigmoid output gate (mla_up_proj_gated)")
    ap.add_argument("--prefill", action="store_true",
                    help="time the MHA-form prefill (mla_prefill) of packed prompts instead of a decode step")
    ap.add_argument("--prefill-seqs", default="4096,4096,4096,4096",
                    help="prompt lengths of the prefill workload (comma separated)")
    ap.add_argument("--prefill-chunk", type=int, default=0,
                    help="with --prefill: chunked prefill, the last N tokens of each prompt are the queries and "
                         "the whole prompt is read from the paged cache (mla_prefill_paged)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="instead of the benchmark, run a plain device copy of this many MiB (5 launches): "
                         "the reference for scaling the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


class TimingEvent:
    """A HIP event for timing only: hipEventDisableSystemFence, recorded on a
    given torch stream (torch's own events carry a system-scope fence, whose
    cache write-back and invalidation stall the next kernel by a few us)."""
    _rt = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if TimingEvent._rt is None:
            rt = ctypes.CDLL("libamdhip64.so.7")   # the HIP runtime torch has loaded
            rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._rt = rt
        self._ct = ctypes
        self._rt = TimingEvent._rt   # kept for __del__ at interpreter exit, when module globals may be gone
        self.h = ctypes.c_void_p()
        self._ok(TimingEvent._rt.hipEventCreateWithFlags(ctypes.byref(self.h), self.DISABLE_SYSTEM_FENCE))

    @staticmethod
    def _ok(code):
        if code != 0:
            raise RuntimeError(f"HIP event call failed with code {code}")

    def record(self, stream):
        self._ok(TimingEvent._rt.hipEventRecord(self.h, self._ct.c_void_p(stream.cuda_stream)))

    def elapsed_time(self, end) -> float:
        ms = self._ct.c_float()
        self._ok(TimingEvent._rt.hipEventElapsedTime(self._ct.byref(ms), self.h, end.h))
        return ms.value

    def __del__(self):
        if getattr(self, "_rt", None) is not None and self.h:
            self._rt.hipEventDestroy(self.h)


def calib_copy(mib):
    import torch
    n = mib * 1024 * 1024
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n, "launches": 5}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every box here has a single MI355X)", file=sys.stderr)
        sys.exit(2)
    if args.calib_copy_mib > 0:
        calib_copy(args.calib_copy_mib)
        return
    if args.prefill:
        bench_prefill(args)
        return
    import torch

    import mla_latent_kv_23_amd as M
    import mla_synth as S

    w = S.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    t0 = time.time()
    inp = S.make_inputs(w, S.SEEDS[w.name])
    d = M.make_dims(n_heads=w.n_heads, d_c=w.d_c, d_rope=w.d_rope, d_nope=w.d_nope, d_v=w.d_v,
                    block_size=w.block_size, softmax_scale=w.softmax_scale, rope_base=w.rope_base,
                    act_dtype=w.act_dtype, cache_dtype=w.cache_dtype)
    B, sq, H = w.batch, w.q_per_seq, w.n_heads
    n_tok = B * sq
    bb = M.cache_block_bytes(d)
    pool = torch.full((inp["n_blocks"] * bb,), 0xFF, dtype=torch.uint8, device=dev)
    table = inp["block_table"].to(dev)
    seqlens = inp["seqlens"].to(dev)
    new_rows = S.new_token_rows(inp, sq)
    hist = torch.ones(inp["c_kv"].shape[0], dtype=torch.bool)
    hist[new_rows] = False
    hist_rows = torch.nonzero(hist)[:, 0]
    # the history is appended once, outside the timed region
    M.append_cache(d, inp["c_kv"][hist_rows].to(dev), inp["k_rope"][hist_rows].to(dev),
                   inp["tok_seq"][hist_rows].to(dev), inp["tok_pos"][hist_rows].to(dev), table, pool)
    step_inputs = dict(
        q_nope=inp["q_nope"].reshape(n_tok, H, -1).to(dev), q_rope=inp["q_rope"].reshape(n_tok, H, -1).to(dev),
        q_pos=S.query_positions(inp["seqlens"], sq).reshape(-1).to(dev),
        new_c_kv=inp["c_kv"][new_rows].to(dev), new_k_rope=inp["k_rope"][new_rows].to(dev),
        new_seq_id=inp["tok_seq"][new_rows].to(dev), new_pos=inp["tok_pos"][new_rows].to(dev),
        block_table=table, seqlens=seqlens, pool=pool, w_uk=inp["w_uk"].to(dev), w_uv=inp["w_uv"].to(dev))
    gate = S.make_gate_logits(w, S.SEEDS[w.name] + 7, n_tok).to(dev) if args.gated else None
    if args.upstream:
        up = S.make_upstream_inputs(w, S.SEEDS[w.name] + 8, n_tok)
        d_cq = up["d_cq"]
        h_new, w_down, w_uq = up["h"].to(dev), up["w_down"].to(dev), up["w_uq"].to(dev)
        c_q = torch.empty((n_tok, d_cq), dtype=h_new.dtype, device=dev)
        ws_down = torch.empty(M.project_down_workspace_bytes(d, n_tok, up["d_model"], d_cq), dtype=torch.uint8,
                              device=dev)
        ws_q = torch.empty(M.absorb_from_latent_workspace_bytes(d, n_tok, d_cq), dtype=torch.uint8, device=dev)
    step = M.DecodeStep(d, B, sq, table.shape[1], num_splits=args.num_splits, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    stream = torch.cuda.current_stream()

    def run_step(ev=None):
        """ev: events recorded before the decode, after it and after the combine, plus (with
        --flush-mib) around the whole step."""
        if args.decode_only:
            if ev:
                ev[0].record(stream)
            M.decode(d, step.q_abs, pool, table, seqlens, args.num_splits, step.workspace, step.o_latent,
                     step.lse, stream=stream)
            if ev:
                ev[1].record(stream)
            if step.needs_combine:
                M.combine(d, seqlens, table.shape[1], step.workspace, step.o_latent, step.lse,
                          args.num_splits, stream=stream)
            if ev:
                ev[2].record(stream)
            return
        if ev and len(ev) > 3:
            ev[3].record(stream)
        dd = step.d
        if args.upstream:
            M.project_down(dd, h_new, w_down, d_cq, step_inputs["new_seq_id"], step_inputs["new_pos"], table, pool,
                           c_q=c_q, workspace=ws_down, stream=stream)
            M.absorb_from_latent(dd, c_q, w_uq, step_inputs["q_pos"], step_inputs["w_uk"],
                                 q_abs=step.q_abs.view(n_tok, H, -1), workspace=ws_q, stream=stream)
        else:   # the absorb and the append of the new tokens in one launch
            M.absorb_append(dd, step_inputs["q_nope"], step_inputs["q_rope"], step_inputs["q_pos"],
                            step_inputs["w_uk"], step_inputs["new_c_kv"], step_inputs["new_k_rope"],
                            step_inputs["new_seq_id"], step_inputs["new_pos"], table, pool,
                            q_abs=step.q_abs.view(n_tok, H, -1), stream=stream)
        if ev:
            ev[0].record(stream)
        M.decode(dd, step.q_abs, pool, table, seqlens, args.num_splits, step.workspace, step.o_latent,
                 step.lse, stream=stream)
        if ev:
            ev[1].record(stream)
        if step.fuse_merge and not args.separate_merge:   # the merge and the up-projection in one launch
            M.combine_up_proj(dd, seqlens, table.shape[1], step.workspace, step.o_latent, step.lse,
                              step_inputs["w_uv"], out=step.out, num_splits=args.num_splits, gate=gate,
                              write_latent=False, stream=stream)
            if ev:
                ev[2].record(stream)
        else:
            if step.needs_combine:
                M.combine(dd, seqlens, table.shape[1], step.workspace, step.o_latent, step.lse, args.num_splits,
                          stream=stream)
            if ev:
                ev[2].record(stream)
            M.up_proj(dd, step.o_latent.view(n_tok, H, -1), step_inputs["w_uv"], out=step.out, stream=stream,
                      gate=gate)
        if ev and len(ev) > 3:
            ev[4].record(stream)

    if args.decode_only:   # the queries must exist once
        M.absorb_q(d, step_inputs["q_nope"], step_inputs["q_rope"], step_inputs["q_pos"], step_inputs["w_uk"],
                   q_abs=step.q_abs.view(n_tok, H, -1), stream=stream)
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    n_ev = 5 if args.flush_mib > 0 else 3
    evs = [tuple(TimingEvent() for _ in range(n_ev)) for _ in range(args.steps)]
    scratch = torch.zeros(args.flush_mib << 18, dtype=torch.float32, device=dev) if args.flush_mib > 0 else None
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        if scratch is not None:         # evicts the cache from the MALL; outside the step's events
            if args.flush_mode == "read":
                scratch.sum()
            else:
                scratch.fill_(float(i & 255))
        run_step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    if scratch is not None:
        ms_step = sum(e[3].elapsed_time(e[4]) for e in evs) / args.steps
    else:
        ms_step = ms_total / args.steps
    dec_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    fused_merge = step.fuse_merge and not args.separate_merge and not args.decode_only
    dec_comb_ms = sum(e[0].elapsed_time(e[2]) for e in evs) / args.steps

    total_tokens = int(inp["seqlens"].to(torch.int64).sum())
    cache_bytes = total_tokens * (bb // w.block_size)              # the cache read once
    visible = sum(int(L) - sq + j + 1 for L in inp["seqlens"].tolist() for j in range(sq))
    flops = visible * H * (2 * (w.d_c + w.d_rope) + 2 * w.d_c)
    dec_gbps = cache_bytes / (dec_ms * 1e-3) / 1e9
    dec_tflops = flops / (dec_ms * 1e-3) / 1e12
    tokens_per_s = n_tok / (ms_step * 1e-3)

    # the decode kernel's bound: the HBM stream unless its flops per cache byte exceed the
    # chip's ridge point (2.5 PFLOP/s / 8 TB/s = 312.5), as with two query rows or an fp8 cache
    mfma_bound = flops / cache_bytes > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    roofline = {"bound": "mfma" if mfma_bound else "hbm",
                "achieved": round(dec_tflops if mfma_bound else dec_gbps, 1),
                "peak": BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBPS,
                "unit": "TFLOP/s" if mfma_bound else "GB/s",
                "frac": round(dec_tflops / BF16_PEAK_TFLOPS if mfma_bound else dec_gbps / HBM_PEAK_GBPS, 4),
                # counter-measured bytes per launch exist for the V3 workload only
                "traffic": measured_traffic() if w.name == "v3_bs64_ctx8k" else None,
                "kernel": "decode576_kernel", "bytes_per_launch": cache_bytes, "flops_per_launch": flops,
                "hbm_frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "mfma_frac": round(dec_tflops / BF16_PEAK_TFLOPS, 4)}

    cpu = None
    if args.cpu_sample_seqs > 0:
        cpu = cpu_baseline(w, inp, args.cpu_sample_seqs)

    rec = {
        "metric": "MLA decode tokens/sec and achieved HBM GB/s (% peak), V3-shape bs64 ctx8k",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.act_dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/sqrt(d_c)) weights)",
        "config": {"workload": w.name, "batch": B, "q_per_seq": sq, "n_heads": H, "d_c": w.d_c,
                   "d_rope": w.d_rope, "d_nope": w.d_nope, "d_v": w.d_v, "seqlen": w.seqlen,
                   "block_size": w.block_size, "cache_dtype": w.cache_dtype, "output_gate": bool(args.gated),
                   "from_hidden_state": bool(args.upstream),
                   "cache_flush_mib": args.flush_mib,
                   **({"cache_flush_mode": args.flush_mode} if args.flush_mib > 0 else {}),
                   "parallelism": "single GPU"},
        "decode_ms": round(dec_ms, 4),
        # from the decode's start to the end of the split merge (with the fused call: of the
        # merge and the up-projection, i.e. the step without the absorb and the append)
        "merge": ("mla_combine_up_proj" if fused_merge else "mla_combine" if step.needs_combine else "none"),
        "decode_combine_ms": round(dec_comb_ms, 4),
        "decode_combine_tokens_per_s": round(n_tok / (dec_comb_ms * 1e-3), 1),
        "decode_hbm_gbps": round(dec_gbps, 1),
        "decode_tflops": round(dec_tflops, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(rec), flush=True)


def bench_prefill(args):
    """Prefill at V3 shape (128 heads) in the MHA form, one call per step:
    whole prompts with mla_prefill (RoPE prep, K/V decompression, causal
    attention), or, with --prefill-chunk N, the last N tokens of each prompt
    attending to the whole prompt in the paged cache with mla_prefill_paged."""
    import torch

    import mla_latent_kv_23_amd as M
    import mla_synth as S

    lens = [int(x) for x in args.prefill_seqs.split(",")]
    chunk = args.prefill_chunk
    w = S.WORKLOADS["v3_bs64_ctx8k"]
    dev = torch.device("cuda:0")
    t0 = time.time()
    d = M.make_dims(n_heads=w.n_heads, d_c=w.d_c, d_rope=w.d_rope, d_nope=w.d_nope, d_v=w.d_v,
                    block_size=w.block_size, softmax_scale=w.softmax_scale, rope_base=w.rope_base,
                    act_dtype=w.act_dtype, cache_dtype=w.cache_dtype)
    H, Tk = w.n_heads, sum(lens)
    qlens = [min(chunk, L) for L in lens] if chunk > 0 else lens
    Tq = sum(qlens)
    stream = torch.cuda.current_stream()
    gate = S.make_gate_logits(w, 4323, Tq).to(dev) if args.gated else None
    out = torch.empty((Tq, H, w.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Tq, H), dtype=torch.float32, device=dev)
    if chunk > 0:
        inp = S.make_chunk_prefill_inputs(w, 4322, torch.tensor(lens, dtype=torch.int32),
                                          torch.tensor(qlens, dtype=torch.int32))
        pool = torch.empty((inp["n_blocks"] * M.cache_block_bytes(d),), dtype=torch.uint8, device=dev)
        table = inp["block_table"].to(dev)
        M.append_cache(d, inp["c_kv"].to(dev), inp["k_rope"].to(dev), inp["tok_seq"].to(dev), inp["tok_pos"].to(dev),
                       table, pool)
        x = {k: inp[k].to(dev) for k in ("q_nope", "q_rope", "w_uk", "w_uv", "cu_q", "cu_k")}
        ws = torch.empty(M.prefill_paged_workspace_bytes(d, Tq, Tk), dtype=torch.uint8, device=dev)

        def step():
            M.prefill_paged(d, x["q_nope"], x["q_rope"], x["cu_q"], max(qlens), x["cu_k"], Tk, pool, table,
                            x["w_uk"], x["w_uv"], workspace=ws, out=out, lse=lse, stream=stream, gate=gate)
    else:
        inp = S.make_prefill_inputs(w, 4321, torch.tensor(lens, dtype=torch.int32))
        x = {k: inp[k].to(dev) for k in ("q_nope", "q_rope", "c_kv", "k_rope", "w_uk", "w_uv", "cu_seqlens")}
        ws = torch.empty(M.prefill_workspace_bytes(d, Tk), dtype=torch.uint8, device=dev)

        def step():
            M.prefill(d, x["q_nope"], x["q_rope"], x["c_kv"], x["k_rope"], x["cu_seqlens"], max(lens), x["w_uk"],
                      x["w_uv"], workspace=ws, out=out, lse=lse, stream=stream, gate=gate)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    start, end = TimingEvent(), TimingEvent()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    # algorithmic FLOPs: causal attention 2 (192 + 128) per visible (query, key) pair and head,
    # plus the K and V decompression 2 x 2 x 512 x 128 per cached token and head
    visible = sum(Lq * (L - Lq) + Lq * (Lq + 1) // 2 for L, Lq in zip(lens, qlens))
    attn_flops = visible * H * 2 * ((w.d_nope + w.d_rope) + w.d_v)
    dec_flops = Tk * H * 2 * 2 * w.d_c * w.d_nope
    tflops = (attn_flops + dec_flops) / (ms * 1e-3) / 1e12
    rec = {
        "metric": ("MLA chunked prefill query tokens/sec (MHA form over the paged cache), V3 shape" if chunk > 0
                   else "MLA prefill prompt tokens/sec (MHA form, causal), V3 shape"),
        "value": round(Tq / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/sqrt(d_c)) weights)",
        "config": {"workload": "prefill_chunk_v3" if chunk > 0 else "prefill_v3", "prompt_lengths": lens,
                   "query_tokens_per_prompt": qlens, "n_heads": H, "d_c": w.d_c, "d_rope": w.d_rope,
                   "d_nope": w.d_nope, "d_v": w.d_v, "output_gate": bool(args.gated), "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "flops_per_step": attn_flops + dec_flops},
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(rec), flush=True)


def cpu_baseline(w, inp, n_seqs):
    """The oracle (non-absorbed, float64) on the first n_seqs sequences, all heads."""
    import numpy as np
    import torch

    from oracle import mla_oracle as O
    seqs = list(range(min(n_seqs, w.batch)))
    t0 = time.time()
    O.decode_batch(inp, q_per_seq=w.q_per_seq, scale=w.softmax_scale, base=w.rope_base,
                   cache_dtype=w.cache_dtype, seqs=seqs)
    dt = time.time() - t0
    try:
        from threadpoolctl import threadpool_info
        cores = max(int(p.get("num_threads", 1)) for p in threadpool_info()) if threadpool_info() else 1
    except Exception:
        cores = torch.get_num_threads()
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(len(seqs) * w.q_per_seq / dt, 4), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": model, "os_cpu_count": os.cpu_count(),
            "torch_threads": torch.get_num_threads(),
            "sample": f"{len(seqs)} of {w.batch} sequences x {w.q_per_seq} query rows, all {w.n_heads} heads, "
                      f"{int(inp['seqlens'][0])} cached tokens each, float64 numpy ({dt:.1f} s)"}


if __name__ == "__main__":
    main()
