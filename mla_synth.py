"""Seeded synthetic inputs for MLA decoding over a paged latent KV cache.

This module only draws numbers and lays out block tables.  It holds none of
the attention arithmetic: no RoPE, no projection, no softmax, no quantiser.
Both the CPU oracle (through the tests) and the GPU path consume exactly the
tensors produced here, so the two never share any computation.

Workloads (shapes and value distributions follow the decode settings used to
discuss MLA in "Transformer升级之路：21、MLA好在哪里？（下）", section 键值共享 /
双重投影: a 512-wide latent plus a 64-wide shared RoPE key, 128 heads of
128 NoPE + 64 RoPE query dims):

  tiny_fp32      fp32, 1 sequence, 1 query, 4 heads, d_c 64, d_R 16,
                 d_nope 32, d_v 32, 128 cached tokens, contiguous blocks
  mid_bf16       bf16, 16 sequences x 4096 tokens, 16 heads, V3 dims,
                 64-token blocks, shuffled block table
  v3_bs64_ctx8k  bf16, 64 sequences x 8192 tokens, 128 heads, V3 dims
  ragged_sq2     bf16, 128 sequences, 2 causal query rows each, lengths
                 uniform in [1024, 32768], random block table
  fp8_ctx64k     bf16 queries, fp8 e4m3 latent cache with per-token fp32
                 scale and bf16 k_R, 32 sequences x 65536 tokens

Value recipe: activations (q_nope, q_R, c_KV, k_R) ~ N(0, 1); W_UK and W_UV
~ N(0, std = 1/sqrt(d_c)) (fan-in of both up-projections is d_c).  Values are
drawn in fp32 with a torch CPU generator and rounded (round-to-nearest-even)
to the activation dtype; every consumer sees the rounded values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    act_dtype: str          # "f32" | "bf16"
    cache_dtype: str        # "f32" | "bf16" | "fp8"
    batch: int
    q_per_seq: int
    n_heads: int
    d_c: int
    d_rope: int
    d_nope: int
    d_v: int
    seqlen: int             # fixed cache length (incl. the new query tokens)
    seqlen_range: Optional[tuple] = None   # (lo, hi) inclusive -> ragged
    block_size: int = 64
    shuffle_blocks: bool = True
    rope_base: float = 10000.0

    @property
    def softmax_scale(self) -> float:
        # 1/sqrt(query-key width): the NoPE part plus the RoPE part.
        return 1.0 / math.sqrt(self.d_nope + self.d_rope)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


V3 = dict(n_heads=128, d_c=512, d_rope=64, d_nope=128, d_v=128)

WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", "f32", "f32", batch=1, q_per_seq=1, n_heads=4, d_c=64,
                          d_rope=16, d_nope=32, d_v=32, seqlen=128, shuffle_blocks=False),
    "mid_bf16": Workload("mid_bf16", "bf16", "bf16", batch=16, q_per_seq=1,
                         **{**V3, "n_heads": 16}, seqlen=4096),
    "v3_bs64_ctx8k": Workload("v3_bs64_ctx8k", "bf16", "bf16", batch=64, q_per_seq=1, **V3,
                              seqlen=8192),
    "ragged_sq2": Workload("ragged_sq2", "bf16", "bf16", batch=128, q_per_seq=2, **V3,
                           seqlen=0, seqlen_range=(1024, 32768)),
    "fp8_ctx64k": Workload("fp8_ctx64k", "bf16", "fp8", batch=32, q_per_seq=1, **V3,
                           seqlen=65536),
}
WORKLOAD_ORDER = ["tiny_fp32", "mid_bf16", "v3_bs64_ctx8k", "ragged_sq2", "fp8_ctx64k"]
SEEDS = {name: 1000 + i for i, name in enumerate(WORKLOAD_ORDER)}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _normal(gen: torch.Generator, shape, std: float = 1.0) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32) * std


def draw_seqlens(w: Workload, gen: torch.Generator) -> torch.Tensor:
    if w.seqlen_range is None:
        return torch.full((w.batch,), w.seqlen, dtype=torch.int32)
    lo, hi = w.seqlen_range
    return torch.randint(lo, hi + 1, (w.batch,), generator=gen, dtype=torch.int64).to(torch.int32)


def make_block_table(seqlens: torch.Tensor, block_size: int, shuffle: bool,
                     gen: torch.Generator, spare_blocks: int = 0):
    """Physical blocks for every sequence; unused table entries are -1.

    Returns (block_table [B, max_blocks] int32, n_phys_blocks).  With
    `shuffle` the physical ids are a random permutation, so logically
    adjacent blocks are scattered through the pool.  `spare_blocks` extra
    physical blocks exist in the pool but are referenced by no sequence.
    """
    nblk = [(int(L) + block_size - 1) // block_size for L in seqlens.tolist()]
    max_blocks = max(nblk) if nblk else 1
    total = sum(nblk)
    n_phys = total + spare_blocks
    ids = torch.randperm(n_phys, generator=gen) if shuffle else torch.arange(n_phys)
    ids = ids[:total].to(torch.int32)
    table = torch.full((len(nblk), max_blocks), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(nblk):
        table[b, :n] = ids[off:off + n]
        off += n
    return table, n_phys


def make_inputs(w: Workload, seed: int, *, spare_blocks: int = 1,
                seqlens: Optional[torch.Tensor] = None) -> dict:
    """Draw one decode step's worth of inputs for workload `w`.

    Keys:
      q_nope [B, s_q, H, d_nope], q_rope [B, s_q, H, d_R]   (act dtype; q_rope unrotated)
      c_kv [T, d_c], k_rope [T, d_R]                        (act dtype; every cached token,
                                                             sequence-major; k_rope unrotated)
      tok_seq [T] int32, tok_pos [T] int32                   (sequence id and position of each token)
      seqlens [B] int32 (cache length incl. the s_q new tokens), cu_seqlens [B+1] int64
      w_uk [H, d_nope, d_c], w_uv [H, d_v, d_c]             (act dtype)
      block_table [B, max_blocks] int32 (-1 = padding), n_blocks (physical pool size)
    """
    gen = torch.Generator().manual_seed(seed)
    if seqlens is None:
        seqlens = draw_seqlens(w, gen)
    seqlens = seqlens.to(torch.int32)
    assert int(seqlens.min()) >= w.q_per_seq, "every sequence holds its own query tokens"
    B, sq, H = len(seqlens), w.q_per_seq, w.n_heads
    dt = TORCH_DTYPE[w.act_dtype]
    T = int(seqlens.sum())
    out = {}
    out["q_nope"] = _normal(gen, (B, sq, H, w.d_nope)).to(dt)
    out["q_rope"] = _normal(gen, (B, sq, H, w.d_rope)).to(dt)
    out["c_kv"] = _normal(gen, (T, w.d_c)).to(dt)
    out["k_rope"] = _normal(gen, (T, w.d_rope)).to(dt)
    std = 1.0 / math.sqrt(w.d_c)
    out["w_uk"] = _normal(gen, (H, w.d_nope, w.d_c), std).to(dt)
    out["w_uv"] = _normal(gen, (H, w.d_v, w.d_c), std).to(dt)
    cu = torch.zeros(B + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(seqlens.to(torch.int64), 0)
    out["seqlens"], out["cu_seqlens"] = seqlens, cu
    out["tok_seq"] = torch.repeat_interleave(torch.arange(B, dtype=torch.int32), seqlens.to(torch.int64))
    out["tok_pos"] = (torch.arange(T, dtype=torch.int64) - cu[:-1].repeat_interleave(seqlens.to(torch.int64))).to(torch.int32)
    table, n_phys = make_block_table(seqlens, w.block_size, w.shuffle_blocks, gen, spare_blocks)
    out["block_table"], out["n_blocks"] = table, n_phys
    return out


def make_prefill_inputs(w: Workload, seed: int, seqlens: torch.Tensor) -> dict:
    """Draw one prefill's worth of packed inputs: every token is both a query
    and a key of its own sequence (same value recipe as make_inputs).

    Keys:
      q_nope [T, H, d_nope], q_rope [T, H, d_R], c_kv [T, d_c], k_rope [T, d_R]  (act dtype, unrotated)
      w_uk [H, d_nope, d_c], w_uv [H, d_v, d_c]                                    (act dtype)
      seqlens [B] int32, cu_seqlens [B+1] int32
    """
    gen = torch.Generator().manual_seed(seed)
    seqlens = seqlens.to(torch.int32)
    H, dt, T = w.n_heads, TORCH_DTYPE[w.act_dtype], int(seqlens.sum())
    out = {}
    out["q_nope"] = _normal(gen, (T, H, w.d_nope)).to(dt)
    out["q_rope"] = _normal(gen, (T, H, w.d_rope)).to(dt)
    out["c_kv"] = _normal(gen, (T, w.d_c)).to(dt)
    out["k_rope"] = _normal(gen, (T, w.d_rope)).to(dt)
    std = 1.0 / math.sqrt(w.d_c)
    out["w_uk"] = _normal(gen, (H, w.d_nope, w.d_c), std).to(dt)
    out["w_uv"] = _normal(gen, (H, w.d_v, w.d_c), std).to(dt)
    cu = torch.zeros(len(seqlens) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(seqlens, 0).to(torch.int32)
    out["seqlens"], out["cu_seqlens"] = seqlens, cu
    return out


def make_chunk_prefill_inputs(w: Workload, seed: int, seqlens: torch.Tensor, qlens: torch.Tensor) -> dict:
    """Chunked prefill over the paged cache: sequence b holds seqlens[b] cached
    tokens (make_inputs' recipe and block tables), of which the last qlens[b]
    are the chunk's queries.  Adds q_nope [Tq, H, d_nope], q_rope [Tq, H, d_R]
    (act dtype, unrotated), cu_q and cu_k [B+1] int32 and qlens [B] int32."""
    seqlens, qlens = seqlens.to(torch.int32), qlens.to(torch.int32)
    assert bool((qlens <= seqlens).all()) and bool((qlens >= 0).all())
    out = make_inputs(w, seed, seqlens=seqlens)
    gen = torch.Generator().manual_seed(seed + 1)
    dt, Tq = TORCH_DTYPE[w.act_dtype], int(qlens.sum())
    out["q_nope"] = _normal(gen, (Tq, w.n_heads, w.d_nope)).to(dt)
    out["q_rope"] = _normal(gen, (Tq, w.n_heads, w.d_rope)).to(dt)
    out["qlens"] = qlens
    cu_q = torch.zeros(len(qlens) + 1, dtype=torch.int32)
    cu_q[1:] = torch.cumsum(qlens, 0).to(torch.int32)
    out["cu_q"], out["cu_k"] = cu_q, out["cu_seqlens"].to(torch.int32)
    return out


# DeepSeek-V3's hidden width and query-latent width (the upstream projections)
V3_D_MODEL, V3_D_CQ = 7168, 1536


def make_upstream_inputs(w: Workload, seed: int, n_tok: int, d_model: int = V3_D_MODEL,
                         d_cq: int = V3_D_CQ) -> dict:
    """Hidden states and upstream projection weights, N(0, 1) activations and
    N(0, 1/sqrt(fan_in)) weights in the act dtype:
      h [n_tok, d_model]; w_down [d_cq + d_c + d_R, d_model] (rows W_DQ, W_DKV, W_KR);
      w_uq [H, d_nope + d_R, d_cq] (per head: the W_UQ rows, then the W_QR rows)."""
    gen = torch.Generator().manual_seed(seed)
    dt = TORCH_DTYPE[w.act_dtype]
    return {
        "h": _normal(gen, (n_tok, d_model)).to(dt),
        "w_down": _normal(gen, (d_cq + w.d_c + w.d_rope, d_model), 1.0 / math.sqrt(d_model)).to(dt),
        "w_uq": _normal(gen, (w.n_heads, w.d_nope + w.d_rope, d_cq), 1.0 / math.sqrt(d_cq)).to(dt),
        "d_model": d_model, "d_cq": d_cq,
    }


def make_gate_logits(w: Workload, seed: int, n_tok: int) -> torch.Tensor:
    """Output-gate logits of gated MLA, [n_tok, H, d_v] in the act dtype, N(0, 1)."""
    gen = torch.Generator().manual_seed(seed)
    return _normal(gen, (n_tok, w.n_heads, w.d_v)).to(TORCH_DTYPE[w.act_dtype])


def new_token_rows(inp: dict, q_per_seq: int) -> torch.Tensor:
    """Indices (into the token arrays) of the last `q_per_seq` tokens of each sequence."""
    cu, L = inp["cu_seqlens"], inp["seqlens"].to(torch.int64)
    start = cu[:-1] + L - q_per_seq
    return (start[:, None] + torch.arange(q_per_seq)[None, :]).reshape(-1)


def query_positions(seqlens: torch.Tensor, q_per_seq: int) -> torch.Tensor:
    """Position of query row j of sequence b: L_b - q_per_seq + j (the new tokens are cached)."""
    L = seqlens.to(torch.int64)
    return (L[:, None] - q_per_seq + torch.arange(q_per_seq)[None, :]).to(torch.int32)
