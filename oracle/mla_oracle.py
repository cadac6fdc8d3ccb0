"""CPU oracle for Multi-head Latent Attention (MLA) decoding over a paged latent cache.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
definition that the GPU library is checked against.  Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it; the product
path never does.  It shares no code, constant or helper with the HIP library.

Everything is numpy float64 unless a storage rounding step says otherwise.

Sources (the web pages this method is described on):
  [P1] "Transformer升级之路：21、MLA好在哪里？（下）" (Su Jianlin) -- sections
       键值共享 (KV sharing: GQA rewritten as a concatenated cache c_i, absorbed
       into W_q / W_o gives an MQA whose K and V are both c), 双重投影 (the
       side-by-side table: training/prefill = MHA with k = c W_k, v = c W_v;
       decoding = MQA with q = x W_q W_k^T, k = v = c, o = [o^(s) W_v^(s)]),
       总而言之 (a shared low-dimensional RoPE key is concatenated to K).
  [P3] "现代 LLM 的 Memory-Compute Trade-off：从 MHA 到 MLA、Sparse 与 Linear
       Attention" -- section "MHA 与 KV Cache" (per-head softmax attention;
       KV size 2 x layers x heads x d_k x tokens x bytes).
  [P4] "DeepSeek-V3 解读：Multi-head Latent Attention" (Chinese translation) --
       sections "RoPE（旋转式位置编码）" (rotate consecutive pairs of
       dimensions by a position-dependent angle), "MLA：高层次的思路" (c^KV =
       W^DKV h, keys/values restored by W^UK, W^UV), "为什么需要解耦 RoPE"
       (extra per-head query part and one shared key get RoPE; only the
       boxed variables -- latent and rotated shared key -- are cached).
  [P2] Tencent Cloud article listing, FlashMLA snippet: decoding runs over a
       paged cache addressed by block_table with per-sequence cache_seqlens
       and returns (o, lse).

Readings where the pages are silent or garbled (each one is a choice):
  R1  softmax scale tau = 1/sqrt(d_nope + d_R) (the pages omit the scale).
  R2  RoPE: interleaved pairs (2i, 2i+1), theta_i = base^(-2i/d_R),
      angle = position * theta_i in float64, cos/sin rounded to float32;
      the rotation (x c - y s, x s + y c) is then formed in float64 (products
      of a <=24-bit input and a float32 cos/sin are exact there).
  R3  cached token t sits at position t; query row j of a sequence with L
      cached tokens (the s_q new ones included) sits at L - s_q + j and sees
      tokens 0..L-s_q+j (causal, bottom-right aligned).
  R4  k_R is cached after rotation, rounded to the cache's k_R dtype
      (float64 -> float32 -> bf16, each round-to-nearest-even).
  R5  fp8 cache: OCP E4M3FN, per-token scale = amax/448 in float32 (amax 0 ->
      scale 1), code = RNE-saturate(float32(c / scale)); the cached latent is
      code * scale.
  R6  weights are stored W_UK [H, d_nope, d_c], W_UV [H, d_v, d_c], so that
      k_C = W_UK[s] c and v = W_UV[s] c.
  R7  lse is the natural log of the sum of exp over the scaled scores.
  R17 upstream projections: c_Q, c_KV and the raw k_R (from h) and q_C, q_R
      (from c_Q) are activations, each rounded once to the act dtype before
      the next step uses it.
  R16 gated MLA: out = sigmoid(g) * o elementwise per head, with the gate
      logits g [tokens, heads, d_v] given (the pages name the gate only).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

F64 = np.float64

# ----------------------------------------------------------------------------
# Rounding helpers (storage precision).  Written from the IEEE-754 / OCP FP8
# definitions; pinned in the tests against torch's own conversions.
# ----------------------------------------------------------------------------


def round_f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of float32 values, round-to-nearest-even."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.ascontiguousarray(x32, dtype=np.float32))
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(F64)


def to_bf16_value(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RNE) -> bf16 (RNE), returned as float64 values."""
    return bf16_bits_to_f64(round_f32_to_bf16_bits(np.asarray(x, dtype=F64).astype(np.float32)))


E4M3_MAX = 448.0


def e4m3fn_encode(v32: np.ndarray) -> np.ndarray:
    """OCP E4M3FN code (uint8) of float32 values, round-to-nearest-even, saturating.

    E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; the
    largest finite magnitude is 448 (exponent 15, mantissa 110); 0x7F/0xFF are
    NaN.  Subnormals have exponent field 0 and value m/8 * 2^-6.
    Implemented by exhaustive nearest search over the 127 non-negative finite
    codes, ties to the even code -- slow but transparently correct.
    """
    v = np.asarray(v32, dtype=np.float32).astype(F64)
    mags = e4m3fn_decode(np.arange(0, 127, dtype=np.uint8))       # 0 .. 448, ascending
    a = np.minimum(np.abs(v), E4M3_MAX)                            # saturate
    idx = np.searchsorted(mags, a)                                 # mags[idx-1] < a <= mags[idx]
    idx = np.clip(idx, 1, 126)
    lo, hi = mags[idx - 1], mags[idx]
    pick_hi = (a - lo > hi - a) | ((a - lo == hi - a) & ((idx % 2) == 0))
    code = np.where(pick_hi, idx, idx - 1).astype(np.uint8)
    code = np.where(a == 0, 0, code).astype(np.uint8)
    sign = np.signbit(v).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


def e4m3fn_decode(code: np.ndarray) -> np.ndarray:
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return (s * val).astype(F64)


def fp8_quantize_token(c_row_values: np.ndarray):
    """Per-token fp8 quantisation of the latent (reading R5).

    c_row_values: [..., d_c] values of the activation (exactly representable in
    float32).  Returns (codes uint8 [..., d_c], scale float32 [...]).
    """
    x32 = np.asarray(c_row_values, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)       # IEEE float32 divide
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    q = (x32 / scale[..., None]).astype(np.float32)                # IEEE float32 divide
    return e4m3fn_encode(q), scale


# ----------------------------------------------------------------------------
# RoPE ([P4] RoPE section; reading R2)
# ----------------------------------------------------------------------------


def rope_cos_sin(pos: np.ndarray, d_rope: int, base: float):
    """cos/sin (float32 values held in float64) of angle pos * base^(-2i/d_rope)."""
    i = np.arange(d_rope // 2, dtype=F64)
    inv_freq = np.power(F64(base), -(2.0 * i) / d_rope)
    ang = np.asarray(pos, dtype=F64)[..., None] * inv_freq
    c = np.cos(ang).astype(np.float32).astype(F64)
    s = np.sin(ang).astype(np.float32).astype(F64)
    return c, s


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate consecutive pairs (x[2i], x[2i+1]) of the last axis by pos*theta_i.

    x: [..., d_rope]; pos broadcastable to x.shape[:-1].  float64 result.
    """
    x = np.asarray(x, dtype=F64)
    d = x.shape[-1]
    c, s = rope_cos_sin(np.broadcast_to(np.asarray(pos), x.shape[:-1]), d, base)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def store_value(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float64 value to a storage dtype and return it as float64."""
    if dtype == "f32":
        return np.asarray(x, dtype=F64).astype(np.float32).astype(F64)
    if dtype == "bf16":
        return to_bf16_value(x)
    raise ValueError(dtype)


def krope_dtype(cache_dtype: str) -> str:
    """dtype the rotated shared key is cached in: fp32 cache -> f32, else bf16."""
    return "f32" if cache_dtype == "f32" else "bf16"


# ----------------------------------------------------------------------------
# What the cache holds for each token ([P4] 为什么需要解耦 RoPE: only the latent
# and the rotated shared key are cached; reading R4/R5)
# ----------------------------------------------------------------------------


def cached_token_values(c_kv: np.ndarray, k_rope_raw: np.ndarray, pos: np.ndarray,
                        cache_dtype: str, base: float):
    """(latent [T, d_c], rotated key [T, d_R]) as stored, returned as float64 values."""
    c = np.asarray(c_kv, dtype=F64)
    if cache_dtype == "fp8":
        codes, scale = fp8_quantize_token(c)
        c = e4m3fn_decode(codes) * scale.astype(F64)[:, None]
    kr = store_value(rope(k_rope_raw, pos, base), krope_dtype(cache_dtype))
    return c, kr


# ----------------------------------------------------------------------------
# Attention ([P1] 双重投影 table, left column = MHA form, right column =
# absorbed MQA form; [P3] MHA 与 KV Cache)
# ----------------------------------------------------------------------------


def _softmax_rows(z: np.ndarray):
    """z [..., n] (-inf allowed) -> (p, lse) with p summing to 1 over the last axis."""
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    Z = np.sum(e, axis=-1, keepdims=True)
    return e / Z, (m + np.log(Z))[..., 0]


def decode_mha_form(q_nope, q_rope, c_cached, kr_cached, q_pos, w_uk, w_uv, scale, base,
                    heads: Optional[Sequence[int]] = None):
    """One sequence, non-absorbed (MHA) form.

    q_nope [s_q, H, d_nope], q_rope [s_q, H, d_R] (unrotated), q_pos [s_q];
    c_cached [L, d_c], kr_cached [L, d_R] (values as cached);
    w_uk [H, d_nope, d_c], w_uv [H, d_v, d_c].
    Per head s: k_C = c W_UK[s]^T and v = c W_UV[s]^T are decompressed
    explicitly, key = [k_C | k_R], query = [q_nope | RoPE(q_R)], and standard
    causal softmax attention runs over tokens t <= position of the query.
    Returns o [s_q, h, d_v], o_lat [s_q, h, d_c], lse [s_q, h] over the chosen heads.
    Nothing is rounded: the rotated query part, the decompressed k_C and v and
    the softmax are exact float64 values.
    """
    q_nope = np.asarray(q_nope, dtype=F64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    s_q, H, _ = q_nope.shape
    L = c_cached.shape[0]
    heads = list(range(H)) if heads is None else list(heads)
    qr = rope(q_rope, q_pos[:, None], base)                              # [s_q, H, d_R]
    c_cached = np.asarray(c_cached, dtype=F64)
    visible = np.arange(L)[None, :] <= q_pos[:, None]                   # [s_q, L]
    o = np.zeros((s_q, len(heads), w_uv.shape[1]))
    o_lat = np.zeros((s_q, len(heads), c_cached.shape[1]))
    lse = np.zeros((s_q, len(heads)))
    for hi, s in enumerate(heads):
        k_c = c_cached @ np.asarray(w_uk[s], dtype=F64).T                 # [L, d_nope]
        v = c_cached @ np.asarray(w_uv[s], dtype=F64).T                   # [L, d_v]
        key = np.concatenate([k_c, kr_cached], axis=1)                    # [L, d_nope + d_R]
        query = np.concatenate([q_nope[:, s, :], qr[:, s, :]], axis=1)    # [s_q, d_nope + d_R]
        z = scale * (query @ key.T)                                       # [s_q, L]
        z = np.where(visible, z, -np.inf)
        p, l = _softmax_rows(z)
        o[:, hi, :] = p @ v
        o_lat[:, hi, :] = p @ c_cached
        lse[:, hi] = l
    return o, o_lat, lse


def prefill_mha_form(q_nope, q_rope, c_kv, k_rope_raw, w_uk, w_uv, scale, base,
                     heads: Optional[Sequence[int]] = None):
    """Prefill of one sequence in the MHA form ([P1] 双重投影, training/prefill
    column: every head attends with k = [c W_UK^T | k_R], v = c W_UV^T).

    All T tokens are both queries and keys: token i sits at position i (R3 with
    an empty history) and sees tokens 0..i.  q_nope [T, H, d_nope], q_rope
    [T, H, d_R] and k_rope_raw [T, d_R] are unrotated; c_kv [T, d_c] is the
    latent as produced (no cache rounding).  The rotated shared key enters the
    attention rounded to bf16, as it is stored in a bf16 cache (R4).
    Returns o [T, h, d_v] and lse [T, h] over the chosen heads.
    """
    T = np.asarray(c_kv).shape[0]
    pos = np.arange(T)
    kr = store_value(rope(k_rope_raw, pos, base), "bf16")
    o, _, lse = decode_mha_form(q_nope, q_rope, np.asarray(c_kv, dtype=F64), kr, pos, w_uk, w_uv, scale, base,
                                heads)
    return o, lse


def prefill_chunk_mha_form(q_nope, q_rope, c_cached, kr_cached, w_uk, w_uv, scale, base,
                           heads: Optional[Sequence[int]] = None):
    """Chunked prefill of one sequence in the MHA form ([P1] 双重投影,
    training/prefill column): its last Lq tokens are the queries and attend to
    all L cached tokens up to their own position (R3: query j at L - Lq + j).
    q_nope [Lq, H, d_nope], q_rope [Lq, H, d_R] (unrotated); c_cached [L, d_c]
    and kr_cached [L, d_R] are the values as cached.  Returns o [Lq, h, d_v]
    and lse [Lq, h]."""
    L, Lq = np.asarray(c_cached).shape[0], np.asarray(q_nope).shape[0]
    q_pos = L - Lq + np.arange(Lq)
    o, _, lse = decode_mha_form(q_nope, q_rope, c_cached, kr_cached, q_pos, w_uk, w_uv, scale, base, heads)
    return o, lse


def absorb_q(q_nope, q_rope, q_pos, w_uk, base):
    """Absorbed query [.., H, d_c + d_R] = [W_UK[s]^T q_nope | RoPE(q_R)] ([P1] 双重投影 right column)."""
    q_nope = np.asarray(q_nope, dtype=F64)
    q_lat = np.einsum("...hn,hnc->...hc", q_nope, np.asarray(w_uk, dtype=F64))
    qr = rope(q_rope, np.asarray(q_pos), base)        # q_pos broadcasts to q_rope.shape[:-1]
    return np.concatenate([q_lat, qr], axis=-1)


# ----------------------------------------------------------------------------
# Upstream projections ([P4] MLA：高层次的思路: the latent c^KV is a
# down-projection of the hidden state h, and queries are compressed to a
# latent c^Q and restored the same way; 为什么需要解耦 RoPE: the RoPE query
# parts come from the query latent and the shared RoPE key from h)
# ----------------------------------------------------------------------------


def project_down(h, w_down, d_cq: int, d_c: int, d_rope: int, out_dtype: Optional[str] = "bf16"):
    """[c_Q | c_KV | k_R] = W_down h for every token, W_down = [W_DQ; W_DKV; W_KR]
    stored [d_cq + d_c + d_R, d_model] (R6's orientation: out = W in).  Reading
    R17: each projection is an activation, stored in the act dtype (rounded
    once from the exact product) before it is used, so the fused path equals
    projecting and then appending.  h [n, d_model].  Returns (c_q, c_kv,
    k_rope_raw) as float64 values."""
    y = np.asarray(h, dtype=F64) @ np.asarray(w_down, dtype=F64).T
    if out_dtype is not None:
        y = store_value(y, out_dtype)
    return y[:, :d_cq], y[:, d_cq:d_cq + d_c], y[:, d_cq + d_c:d_cq + d_c + d_rope]


def query_from_latent(c_q, w_uq, q_pos, w_uk, d_nope: int, base: float, out_dtype: Optional[str] = "bf16"):
    """Absorbed queries from the query latent: per head s, [q_C | q_R] = W_UQ[s] c_Q
    (W_UQ [H, d_nope + d_R, d_cq]: the W^UQ rows, then the W^QR rows), stored
    in the act dtype (R17), then absorb_q.  c_q [n, d_cq], q_pos [n].
    Returns q_abs [n, H, d_c + d_R] (float64)."""
    q = np.einsum("tk,hrk->thr", np.asarray(c_q, dtype=F64), np.asarray(w_uq, dtype=F64))
    if out_dtype is not None:
        q = store_value(q, out_dtype)
    return absorb_q(q[..., :d_nope], q[..., d_nope:], np.asarray(q_pos)[:, None], w_uk, base)


def decode_absorbed_form(q_abs, c_cached, kr_cached, q_pos, scale):
    """One sequence, absorbed (KV-shared MQA) form over the latent cache.

    q_abs [s_q, H, d_c + d_R]; every head uses key [c | k_R] (d_c + d_R wide)
    and value c (the first d_c entries of the key).
    Returns o_lat [s_q, H, d_c], lse [s_q, H].
    """
    q_abs = np.asarray(q_abs, dtype=F64)
    L, d_c = c_cached.shape
    key = np.concatenate([c_cached, kr_cached], axis=1)                  # [L, d_c + d_R]
    z = scale * np.einsum("jhk,tk->jht", q_abs, key)                     # [s_q, H, L]
    visible = np.arange(L)[None, :] <= np.asarray(q_pos)[:, None]
    z = np.where(visible[:, None, :], z, -np.inf)
    p, lse = _softmax_rows(z)
    return p @ c_cached, lse


def up_proj(o_lat, w_uv):
    """o[.., s, :] = W_UV[s] o_lat[.., s, :] ([P1] 双重投影: o = [o^(1) W_v^(1), ...])."""
    return np.einsum("...hc,hvc->...hv", np.asarray(o_lat, dtype=F64), np.asarray(w_uv, dtype=F64))


def output_gate(o, gate_logits):
    """Gated MLA: each head's attention output is scaled elementwise by a
    logistic gate, o * 1 / (1 + e^-g) ([P1], reader comments: gated MLA is MLA
    with an output gate).  Reading R16: the gate logits g have o's shape and are
    an input (computed upstream from the hidden state)."""
    o = np.asarray(o, dtype=F64)
    g = np.asarray(gate_logits, dtype=F64)
    # the logistic function in the form that never overflows: for g >= 0,
    # 1 / (1 + e^-g); for g < 0, e^g / (1 + e^g)
    e = np.exp(-np.abs(g))
    sig = np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return o * sig


def lse_merge(o_parts: Sequence[np.ndarray], lse_parts: Sequence[np.ndarray]):
    """Merge attention over disjoint key sets: lse = log sum exp(lse_k), o = sum e^(lse_k - lse) o_k.

    A part with lse = -inf (no keys) carries zero weight.
    """
    L = np.stack([np.asarray(x, dtype=F64) for x in lse_parts])          # [K, ...]
    m = np.max(L, axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(L - m_safe)
    tot = np.sum(w, axis=0)
    lse = m_safe + np.log(tot)
    o = sum(wk[..., None] * np.asarray(ok, dtype=F64) for wk, ok in zip(w, o_parts)) / tot[..., None]
    return o, lse


# ----------------------------------------------------------------------------
# Batch driver over the synthetic inputs (float64 throughout)
# ----------------------------------------------------------------------------


def decode_batch(inp: dict, *, q_per_seq: int, scale: float, base: float, cache_dtype: str,
                 seqs: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None,
                 form: str = "mha"):
    """Reference outputs for the chosen sequences (default: all).

    inp holds numpy (or torch CPU) arrays as produced by the input generator:
    q_nope, q_rope, c_kv, k_rope, seqlens, cu_seqlens, w_uk, w_uv.
    Returns dict with o [b, s_q, h, d_v], o_lat [b, s_q, h, d_c], lse [b, s_q, h].
    """
    a = {}
    for k, v in inp.items():
        if hasattr(v, "is_floating_point"):            # torch CPU tensor
            v = v.double().numpy() if v.is_floating_point() else v.numpy()
        a[k] = v
    seqlens = np.asarray(a["seqlens"], dtype=np.int64)
    cu = np.asarray(a["cu_seqlens"], dtype=np.int64)
    seqs = list(range(len(seqlens))) if seqs is None else list(seqs)
    H = a["q_nope"].shape[2]
    heads_l = list(range(H)) if heads is None else list(heads)
    outs = {"o": [], "o_lat": [], "lse": []}
    for b in seqs:
        L = int(seqlens[b])
        c_raw = a["c_kv"][cu[b]:cu[b] + L]
        kr_raw = a["k_rope"][cu[b]:cu[b] + L]
        c_cached, kr_cached = cached_token_values(c_raw, kr_raw, np.arange(L), cache_dtype, base)
        q_pos = L - q_per_seq + np.arange(q_per_seq)
        if form == "mha":
            o, o_lat, lse = decode_mha_form(a["q_nope"][b], a["q_rope"][b], c_cached, kr_cached,
                                            q_pos, a["w_uk"], a["w_uv"], scale, base, heads_l)
        else:
            q_abs = absorb_q(a["q_nope"][b][:, heads_l], a["q_rope"][b][:, heads_l],
                             q_pos[:, None] * np.ones((1, len(heads_l)), dtype=np.int64),
                             np.asarray(a["w_uk"])[heads_l], base)
            o_lat, lse = decode_absorbed_form(q_abs, c_cached, kr_cached, q_pos, scale)
            o = up_proj(o_lat, np.asarray(a["w_uv"])[heads_l])
        outs["o"].append(o)
        outs["o_lat"].append(o_lat)
        outs["lse"].append(lse)
    return {k: np.stack(v) for k, v in outs.items()}


# ----------------------------------------------------------------------------
# Paged cache append ([P4] 为什么需要解耦 RoPE: what is cached; [P2] FlashMLA
# snippet: block_table addressing).  Expected pool bytes, derived from the
# layout definition with plain integer arithmetic.
# ----------------------------------------------------------------------------


def block_bytes(block_size: int, d_c: int, d_rope: int, cache_dtype: str) -> int:
    if cache_dtype == "f32":
        return block_size * (d_c + d_rope) * 4
    if cache_dtype == "bf16":
        return block_size * (d_c + d_rope) * 2
    if cache_dtype == "fp8":
        return block_size * d_c + block_size * 4 + block_size * d_rope * 2
    raise ValueError(cache_dtype)


def kv_bytes_per_token(d_c: int, d_rope: int, cache_dtype: str) -> int:
    """Latent cache bytes per token and layer: (d_c + d_R) * element size (fp8: codes + scale + bf16 k_R)."""
    return block_bytes(1, d_c, d_rope, cache_dtype)


def mha_kv_elements_per_token(n_layers: int, n_heads: int, d_k: int) -> int:
    """Plain MHA cache: K and V for every head and layer ([P3] MHA 与 KV Cache)."""
    return 2 * n_layers * n_heads * d_k


def append_expected_pool(pool_bytes: np.ndarray, c_kv, k_rope_raw, seq_id, pos, block_table,
                         *, block_size: int, d_c: int, d_rope: int, cache_dtype: str, base: float):
    """Return a copy of `pool_bytes` (uint8, whole pool) with the tokens written.

    Token n of sequence seq_id[n] at position pos[n] goes to physical block
    block_table[seq, pos // block_size], slot pos % block_size.  The stored
    payload is [c | RoPE(k_R, pos)] at the cache dtype; for fp8 the block is
    [codes (block_size x d_c) | scales (block_size fp32) | k_R (block_size x d_R bf16)].
    """
    out = np.array(pool_bytes, dtype=np.uint8, copy=True)
    c = np.asarray(c_kv, dtype=F64)
    kr = rope(k_rope_raw, np.asarray(pos, dtype=np.int64), base)
    bt = np.asarray(block_table, dtype=np.int64)
    bb = block_bytes(block_size, d_c, d_rope, cache_dtype)
    if cache_dtype == "fp8":
        codes, scale = fp8_quantize_token(c)
        kr_bits = round_f32_to_bf16_bits(kr.astype(np.float32))
    for n in range(c.shape[0]):
        p = int(pos[n])
        blk = int(bt[int(seq_id[n]), p // block_size])
        slot = p % block_size
        base_off = blk * bb
        if cache_dtype == "f32":
            row = np.concatenate([c[n], kr[n]]).astype(np.float32).view(np.uint8)
            off = base_off + slot * (d_c + d_rope) * 4
            out[off:off + row.size] = row
        elif cache_dtype == "bf16":
            row = round_f32_to_bf16_bits(np.concatenate([c[n], kr[n]]).astype(np.float32)).view(np.uint8)
            off = base_off + slot * (d_c + d_rope) * 2
            out[off:off + row.size] = row
        else:
            off = base_off + slot * d_c
            out[off:off + d_c] = codes[n]
            off = base_off + block_size * d_c + slot * 4
            out[off:off + 4] = np.array([scale[n]], dtype=np.float32).view(np.uint8)
            off = base_off + block_size * d_c + block_size * 4 + slot * d_rope * 2
            out[off:off + d_rope * 2] = kr_bits[n].view(np.uint8)
    return out


def softmax_scale(d_nope: int, d_rope: int) -> float:
    """Reading R1: 1/sqrt(width of the query-key product)."""
    return 1.0 / math.sqrt(d_nope + d_rope)
