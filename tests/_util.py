"""Shared helpers for the parity tests: workload -> dims, pool builders,
tolerance checks.  The expected side always comes from the CPU oracle."""
from __future__ import annotations

import json
import math
import os
import sys

import numpy as np
import torch

import mla_synth as S
from oracle import mla_oracle as O

# Tolerances: bf16 paths max-abs <= 1e-2 and relative L2 <= 5e-3; fp32 paths
# relative L2 <= 1e-5.
BF16_MAX_ABS, BF16_REL_L2, F32_REL_L2 = 1e-2, 5e-3, 1e-5


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dims_of(w: S.Workload):
    import mla_latent_kv_23_amd as M
    return M.make_dims(n_heads=w.n_heads, d_c=w.d_c, d_rope=w.d_rope, d_nope=w.d_nope, d_v=w.d_v,
                       block_size=w.block_size, softmax_scale=w.softmax_scale, rope_base=w.rope_base,
                       act_dtype=w.act_dtype, cache_dtype=w.cache_dtype)


def errors_full(got, want, out_dtype: str = "f32"):
    """(max-abs, rel-L2, raw max-abs) of got vs the exact value.  For a bf16
    output the first max-abs excludes the output format's own representation
    error (half a bf16 ulp of the exact value, 2^-8 |want| at most), which alone
    exceeds 1e-2 once |want| > 2.56; the raw max-abs excludes nothing.  For
    float32 outputs the two are the same."""
    g = got.detach().double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    w = np.asarray(want, dtype=np.float64)
    assert g.shape == w.shape, (g.shape, w.shape)
    assert np.all(np.isfinite(g)), "non-finite output"
    err = g - w
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(w), 1e-300))
    repr_err = np.ldexp(np.abs(w), -8) if out_dtype == "bf16" else 0.0
    mx = float(np.max(np.maximum(np.abs(err) - repr_err, 0.0))) if err.size else 0.0
    raw = float(np.max(np.abs(err))) if err.size else 0.0
    return mx, rel, raw


def errors(got, want, out_dtype: str = "f32"):
    """(max-abs beyond the output's representation error, rel-L2); see errors_full."""
    mx, rel, _ = errors_full(got, want, out_dtype)
    return mx, rel


def log_errors(what: str, mx: float, rel: float, raw: float):
    """Append one comparison to the file named by MLA_ERR_LOG (if set): the
    measured errors the design notes quote."""
    path = os.environ.get("MLA_ERR_LOG")
    if path:
        test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
        with open(path, "a") as f:
            f.write(json.dumps({"test": test, "what": what, "max_abs": mx, "max_abs_raw": raw, "rel_l2": rel}) + "\n")


def assert_close(got, want, act_dtype: str, what: str):
    out_dtype = "f32" if (isinstance(got, torch.Tensor) and got.dtype == torch.float32) else act_dtype
    mx, rel, raw = errors_full(got, want, out_dtype)
    log_errors(what, mx, rel, raw)
    if act_dtype == "f32":
        assert rel <= F32_REL_L2, f"{what}: rel-L2 {rel:.3e} > {F32_REL_L2} (max-abs {raw:.3e})"
    else:
        assert mx <= BF16_MAX_ABS and rel <= BF16_REL_L2, \
            f"{what}: max-abs {mx:.3e} beyond the output's half ulp (raw {raw:.3e}), rel-L2 {rel:.3e}"
    return mx, rel


def assert_close_ulp(got, want, act_dtype: str, what: str, ulps: float = 1.5):
    """Intermediate tensors stored in the activation dtype (q_abs): each element
    is the exact value rounded once to that dtype, up to `ulps` units in the last
    place (float32 accumulation order may move a rounding by one unit); the
    whole tensor must also meet the relative-L2 bar."""
    g = got.detach().double().cpu().numpy()
    w = np.asarray(want, dtype=np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    mant = 7 if act_dtype == "bf16" else 23
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(w), 1e-30))) - mant)
    tol = ulps * ulp + 1e-6 * float(np.max(np.abs(w)))
    bad = np.abs(g - w) > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond {ulps} ulp"
    _, rel = errors(got, want)
    assert rel <= (F32_REL_L2 if act_dtype == "f32" else BF16_REL_L2), f"{what}: rel-L2 {rel:.3e}"


def to_act(x: np.ndarray, act_dtype: str, device) -> torch.Tensor:
    """Round an oracle float64 array to the activation dtype (RNE) on the device."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.float32)
    return t.to(S.TORCH_DTYPE[act_dtype]).to(device)


def new_tokens(inp: dict, q_per_seq: int):
    rows = S.new_token_rows(inp, q_per_seq)
    return rows


def oracle_pool_bytes(w: S.Workload, inp: dict, poison: int, rows=None) -> np.ndarray:
    """Expected pool after appending `rows` (default: every token) into a poisoned pool."""
    bb = O.block_bytes(w.block_size, w.d_c, w.d_rope, w.cache_dtype)
    pool = np.full(inp["n_blocks"] * bb, poison, dtype=np.uint8)
    rows = np.arange(inp["c_kv"].shape[0]) if rows is None else np.asarray(rows)
    return O.append_expected_pool(
        pool, inp["c_kv"][rows].double().numpy(), inp["k_rope"][rows].double().numpy(),
        inp["tok_seq"][rows].numpy(), inp["tok_pos"][rows].numpy(), inp["block_table"].numpy(),
        block_size=w.block_size, d_c=w.d_c, d_rope=w.d_rope, cache_dtype=w.cache_dtype, base=w.rope_base)


def gpu_pool(w: S.Workload, inp: dict, device, poison: int = 0xFF, rows=None) -> torch.Tensor:
    """Pool filled by the library's own append call (all tokens, or `rows`)."""
    import mla_latent_kv_23_amd as M
    d = dims_of(w)
    bb = M.cache_block_bytes(d)
    pool = torch.full((inp["n_blocks"] * bb,), poison, dtype=torch.uint8, device=device)
    sel = slice(None) if rows is None else torch.as_tensor(rows)
    M.append_cache(d, inp["c_kv"][sel].to(device), inp["k_rope"][sel].to(device),
                   inp["tok_seq"][sel].to(device), inp["tok_pos"][sel].to(device),
                   inp["block_table"].to(device), pool)
    return pool


def q_positions_flat(inp: dict, q_per_seq: int) -> torch.Tensor:
    return S.query_positions(inp["seqlens"], q_per_seq).reshape(-1)
