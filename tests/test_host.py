"""Host-side logic that needs no GPU: the benchmark's refusal of several GPUs,
its reading of the committed counter summary, and the input generators of the
prefill and upstream workloads."""
import os
import subprocess
import sys

import torch

import mla_synth as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_reads_the_committed_traffic_summary():
    sys.path.insert(0, ROOT)
    import bench
    # the summary under profiles/ was taken on the current decode sources
    assert bench.measured_traffic() is not None
    assert 600_000_000 < bench.measured_traffic() < 800_000_000


def test_chunk_prefill_inputs_are_consistent():
    w = S.WORKLOADS["v3_bs64_ctx8k"].replace(n_heads=4)
    inp = S.make_chunk_prefill_inputs(w, 3, torch.tensor([100, 7, 64], dtype=torch.int32),
                                      torch.tensor([10, 7, 0], dtype=torch.int32))
    assert inp["cu_q"].tolist() == [0, 10, 17, 17]
    assert inp["cu_k"].tolist() == [0, 100, 107, 171]
    assert inp["q_nope"].shape == (17, 4, w.d_nope) and inp["q_rope"].shape == (17, 4, w.d_rope)
    assert inp["c_kv"].shape == (171, w.d_c)
    # every cached token has a block in its sequence's table
    tbl = inp["block_table"]
    for sq, p in zip(inp["tok_seq"].tolist(), inp["tok_pos"].tolist()):
        assert tbl[sq, p // w.block_size] >= 0


def test_upstream_inputs_shapes_and_scale():
    w = S.WORKLOADS["v3_bs64_ctx8k"].replace(n_heads=8)
    up = S.make_upstream_inputs(w, 4, 5, d_model=256, d_cq=64)
    assert up["h"].shape == (5, 256)
    assert up["w_down"].shape == (64 + w.d_c + w.d_rope, 256)
    assert up["w_uq"].shape == (8, w.d_nope + w.d_rope, 64)
    # N(0, 1/sqrt(fan_in)) weights
    assert abs(up["w_down"].float().std().item() * 16 - 1) < 0.05
    assert abs(up["w_uq"].float().std().item() * 8 - 1) < 0.05
