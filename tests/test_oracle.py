"""Pins for the CPU oracle: every check here ties the oracle to something other
than itself -- a library routine, a closed form, an invariant the pages state,
a special case with a known answer, or brute force on tiny inputs.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
import mla_synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- rounding pins

def test_bf16_rounding_matches_torch():
    r = _rng(1)
    x = np.concatenate([
        r.standard_normal(20000).astype(np.float32) * 10,
        # exact ties: low 16 bits == 0x8000, both parities of bit 16
        (np.arange(2000, dtype=np.uint32) * 0x10000 + 0x3F808000).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.3e38, -3.3e38], dtype=np.float32),
    ])
    ours = O.round_f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3fn_decode_matches_torch():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(O.e4m3fn_decode(codes), ref)


def test_e4m3fn_encode_matches_torch_cast():
    r = _rng(2)
    mags = O.e4m3fn_decode(np.arange(127, dtype=np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2                       # exact ties between neighbours
    x = np.concatenate([
        r.standard_normal(50000) * 100, r.uniform(-448, 448, 50000), r.standard_normal(5000) * 1e-3,
        mids, -mids, mags, -mags, [448.0, -448.0, 0.0],
    ]).astype(np.float32)
    ours = O.e4m3fn_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_fp8_token_quantiser_properties():
    r = _rng(3)
    c = torch.from_numpy(r.standard_normal((64, 512)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    c[5] = 0.0
    codes, scale = O.fp8_quantize_token(c)
    assert scale.dtype == np.float32 and scale[5] == 1.0 and not codes[5].any()
    amax = np.abs(c).max(-1)
    for t in range(64):
        if t == 5:
            continue
        assert scale[t] == np.float32(amax[t]) / np.float32(448.0)
        j = int(np.argmax(np.abs(c[t])))
        assert (codes[t, j] & 0x7F) == 0x7E                  # the largest element maps to +-448
    deq = O.e4m3fn_decode(codes) * scale[:, None]
    # E4M3 has 3 mantissa bits: relative error <= 2^-4 for normals, absolute <= 2^-10*scale below
    err = np.abs(deq - c)
    bound = np.maximum(np.abs(c) * 2.0 ** -4, scale[:, None] * 2.0 ** -10)
    assert np.all(err <= bound + 1e-12)


# ---------------------------------------------------------------- RoPE pins

def test_rope_identity_at_position_zero():
    x = _rng(4).standard_normal((7, 64))
    assert np.array_equal(O.rope(x, np.zeros(7, dtype=np.int64), 10000.0), x)


def test_rope_single_pair_is_complex_rotation():
    # d_R = 2: theta_0 = base^0 = 1, so position p rotates (x, y) by p radians.
    r = _rng(5)
    xy = r.standard_normal((50, 2))
    pos = r.integers(0, 70000, 50)
    got = O.rope(xy, pos, 10000.0)
    z = (xy[:, 0] + 1j * xy[:, 1]) * np.exp(1j * pos.astype(np.float64))
    assert np.allclose(got[:, 0], z.real, atol=1e-6) and np.allclose(got[:, 1], z.imag, atol=1e-6)


def test_rope_frequency_ladder():
    # d_R = 4, base 10000: pair 0 turns by p, pair 1 by p * 10000^(-1/2) = p / 100.
    x = np.array([[1.0, 0.0, 1.0, 0.0]])
    for p in [1, 7, 100, 12345]:
        got = O.rope(x, np.array([p]), 10000.0)[0]
        assert abs(math.atan2(got[1], got[0]) - math.remainder(p, 2 * math.pi)) < 1e-6
        assert abs(math.atan2(got[3], got[2]) - math.remainder(p / 100.0, 2 * math.pi)) < 1e-6


def test_rope_preserves_norm_and_is_relative():
    r = _rng(6)
    q, k = r.standard_normal((2, 64))
    for m, n, d in [(5, 3, 11), (1000, 20, 777), (65535, 0, 5)]:
        a = O.rope(q[None], np.array([m]), 10000.0)[0] @ O.rope(k[None], np.array([n]), 10000.0)[0]
        b = O.rope(q[None], np.array([m + d]), 10000.0)[0] @ O.rope(k[None], np.array([n + d]), 10000.0)[0]
        assert abs(a - b) < 1e-4 * (1 + abs(a))
        assert abs(np.linalg.norm(O.rope(q[None], np.array([m]), 10000.0)) - np.linalg.norm(q)) < 1e-5


# ---------------------------------------------------------------- attention pins

def _tiny_problem(seed, L=9, s_q=1, H=3, d_c=8, d_R=4, d_nope=5, d_v=6):
    r = _rng(seed)
    return dict(
        q_nope=r.standard_normal((s_q, H, d_nope)), q_rope=r.standard_normal((s_q, H, d_R)),
        c=r.standard_normal((L, d_c)), kr=r.standard_normal((L, d_R)),
        w_uk=r.standard_normal((H, d_nope, d_c)) / math.sqrt(d_c),
        w_uv=r.standard_normal((H, d_v, d_c)) / math.sqrt(d_c),
        q_pos=np.arange(L - s_q, L), scale=1.0 / math.sqrt(d_nope + d_R), base=10000.0)


def _brute_force(P):
    """Pure-Python loops over the MHA form: decompress each key/value, exp-sum."""
    s_q, H, d_nope = P["q_nope"].shape
    L, d_c = P["c"].shape
    d_R = P["kr"].shape[1]
    d_v = P["w_uv"].shape[1]
    o = np.zeros((s_q, H, d_v)); lse = np.zeros((s_q, H))
    for j in range(s_q):
        p = int(P["q_pos"][j])
        ang = [p * P["base"] ** (-2.0 * i / d_R) for i in range(d_R // 2)]
        for s in range(H):
            qr = []
            for i in range(d_R // 2):
                cs, sn = float(np.float32(math.cos(ang[i]))), float(np.float32(math.sin(ang[i])))
                x, y = P["q_rope"][j, s, 2 * i], P["q_rope"][j, s, 2 * i + 1]
                qr += [x * cs - y * sn, x * sn + y * cs]
            z = []
            for t in range(p + 1):
                k_c = [sum(P["w_uk"][s, n, c] * P["c"][t, c] for c in range(d_c)) for n in range(d_nope)]
                dot = sum(P["q_nope"][j, s, n] * k_c[n] for n in range(d_nope))
                dot += sum(qr[i] * P["kr"][t, i] for i in range(d_R))
                z.append(P["scale"] * dot)
            m = max(z)
            den = sum(math.exp(zz - m) for zz in z)
            lse[j, s] = m + math.log(den)
            for e in range(d_v):
                num = 0.0
                for t in range(p + 1):
                    v = sum(P["w_uv"][s, e, c] * P["c"][t, c] for c in range(d_c))
                    num += math.exp(z[t] - m) * v
                o[j, s, e] = num / den
    return o, lse


@pytest.mark.parametrize("s_q,L", [(1, 9), (2, 9), (2, 2), (1, 1)])
def test_mha_form_matches_brute_force(s_q, L):
    P = _tiny_problem(10 + s_q + L, L=L, s_q=s_q)
    o, o_lat, lse = O.decode_mha_form(P["q_nope"], P["q_rope"], P["c"], P["kr"], P["q_pos"],
                                      P["w_uk"], P["w_uv"], P["scale"], P["base"])
    o_bf, lse_bf = _brute_force(P)
    assert np.allclose(o, o_bf, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, lse_bf, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("s_q", [1, 2])
def test_absorbed_equals_non_absorbed(s_q):
    # The pages state the two forms are the same function of the inputs.
    P = _tiny_problem(20 + s_q, L=40, s_q=s_q, H=5, d_c=32, d_R=8, d_nope=16, d_v=12)
    o, o_lat, lse = O.decode_mha_form(P["q_nope"], P["q_rope"], P["c"], P["kr"], P["q_pos"],
                                      P["w_uk"], P["w_uv"], P["scale"], P["base"])
    q_abs = O.absorb_q(P["q_nope"], P["q_rope"], P["q_pos"][:, None] * np.ones((1, 5), np.int64),
                       P["w_uk"], P["base"])
    o_lat2, lse2 = O.decode_absorbed_form(q_abs, P["c"], P["kr"], P["q_pos"], P["scale"])
    o2 = O.up_proj(o_lat2, P["w_uv"])
    assert np.allclose(o2, o, rtol=1e-11, atol=1e-12)
    assert np.allclose(o_lat2, o_lat, rtol=1e-11, atol=1e-12)
    assert np.allclose(lse2, lse, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("groups", [1, 2, 4])
def test_selection_matrices_reduce_to_gqa(groups):
    """With c = [k^(1..g) | v^(1..g)] and W_UK/W_UV picking head s's group, MLA is
    textbook GQA (g=1: MQA); compared against torch's scaled_dot_product_attention."""
    r = _rng(30 + groups)
    H, d_k, d_v, L, s_q, d_R = 8, 16, 16, 37, 2, 2
    hpg = H // groups
    d_c = groups * (d_k + d_v)
    c = r.standard_normal((L, d_c))
    w_uk = np.zeros((H, d_k, d_c)); w_uv = np.zeros((H, d_v, d_c))
    for s in range(H):
        g = s // hpg
        w_uk[s, :, g * d_k:(g + 1) * d_k] = np.eye(d_k)
        w_uv[s, :, groups * d_k + g * d_v:groups * d_k + (g + 1) * d_v] = np.eye(d_v)
    q = r.standard_normal((s_q, H, d_k))
    zr = np.zeros((L, d_R))
    q_pos = np.arange(L - s_q, L)
    scale = 1.0 / math.sqrt(d_k + d_R)
    o, _, lse = O.decode_mha_form(q, np.zeros((s_q, H, d_R)), c, zr, q_pos, w_uk, w_uv, scale, 10000.0)
    K = torch.from_numpy(c[:, :groups * d_k].reshape(L, groups, d_k).transpose(1, 0, 2).copy())
    V = torch.from_numpy(c[:, groups * d_k:].reshape(L, groups, d_v).transpose(1, 0, 2).copy())
    K = K.repeat_interleave(hpg, 0); V = V.repeat_interleave(hpg, 0)
    Q = torch.from_numpy(q.transpose(1, 0, 2).copy())
    mask = torch.from_numpy(np.arange(L)[None, :] <= q_pos[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
    assert np.allclose(o, ref.numpy().transpose(1, 0, 2), rtol=1e-10, atol=1e-12)


def test_two_causal_queries_equal_two_single_decodes():
    P = _tiny_problem(40, L=30, s_q=2, H=4, d_c=16, d_R=4, d_nope=8, d_v=8)
    o2, ol2, lse2 = O.decode_mha_form(P["q_nope"], P["q_rope"], P["c"], P["kr"], P["q_pos"],
                                      P["w_uk"], P["w_uv"], P["scale"], P["base"])
    for j, L in [(0, 29), (1, 30)]:
        o1, ol1, lse1 = O.decode_mha_form(P["q_nope"][j:j + 1], P["q_rope"][j:j + 1], P["c"][:L],
                                          P["kr"][:L], np.array([L - 1]), P["w_uk"], P["w_uv"],
                                          P["scale"], P["base"])
        assert np.allclose(o1[0], o2[j], rtol=1e-13, atol=1e-14)
        assert np.allclose(lse1[0], lse2[j], rtol=1e-13, atol=1e-14)


def test_split_invariance_of_lse_merge():
    r = _rng(50)
    L, H, d_c, d_R = 100, 6, 16, 4
    q_abs = r.standard_normal((1, H, d_c + d_R))
    c, kr = r.standard_normal((L, d_c)), r.standard_normal((L, d_R))
    full_o, full_lse = O.decode_absorbed_form(q_abs, c, kr, np.array([L - 1]), 0.3)
    for cuts in [[0, 100], [0, 1, 100], [0, 37, 64, 99, 100], [0, 50, 50, 100]]:
        parts_o, parts_l = [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            if b == a:       # an empty split: no keys, lse = -inf, output zero
                parts_o.append(np.zeros_like(full_o)); parts_l.append(np.full(full_lse.shape, -np.inf))
                continue
            o, l = O.decode_absorbed_form(q_abs, c[a:b], kr[a:b], np.array([b - a - 1]), 0.3)
            parts_o.append(o); parts_l.append(l)
        mo, ml = O.lse_merge(parts_o, parts_l)
        assert np.allclose(mo, full_o, rtol=1e-12, atol=1e-13) and np.allclose(ml, full_lse, rtol=1e-13)


def test_single_token_returns_its_value():
    P = _tiny_problem(60, L=1, s_q=1)
    o, o_lat, lse = O.decode_mha_form(P["q_nope"], P["q_rope"], P["c"], P["kr"], P["q_pos"],
                                      P["w_uk"], P["w_uv"], P["scale"], P["base"])
    for s in range(P["q_nope"].shape[1]):
        assert np.allclose(o_lat[0, s], P["c"][0], rtol=1e-15)
        assert np.allclose(o[0, s], P["w_uv"][s] @ P["c"][0], rtol=1e-13)


def test_zero_query_gives_uniform_mean():
    P = _tiny_problem(61, L=23, s_q=1)
    P["q_nope"][:] = 0; P["q_rope"][:] = 0
    o, o_lat, lse = O.decode_mha_form(P["q_nope"], P["q_rope"], P["c"], P["kr"], P["q_pos"],
                                      P["w_uk"], P["w_uv"], P["scale"], P["base"])
    assert np.allclose(o_lat[0], P["c"].mean(0)[None, :], rtol=1e-13, atol=1e-14)
    assert np.allclose(lse, math.log(23), rtol=1e-14)


def test_softmax_scale_is_inverse_sqrt_qk_width():
    assert O.softmax_scale(128, 64) == 1.0 / math.sqrt(192)
    assert O.softmax_scale(32, 16) == 1.0 / math.sqrt(48)


# ---------------------------------------------------------------- size pins (golden)

def test_kv_size_figures_from_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "kv_size_figures.json")))
    a = g["mla_vs_gqa_groups"]
    elems = a["d_c"] + a["d_rope"]
    assert elems == a["groups"] * 2 * a["head_dim"] == 576
    assert O.kv_bytes_per_token(a["d_c"], a["d_rope"], "bf16") == 2 * elems == 1152
    b = g["mla_vs_gqa8_128"]
    ratio = (b["d_c"] + b["d_rope"]) / O.mha_kv_elements_per_token(1, b["gqa_groups"], b["head_dim"])
    assert ratio == 0.28125 and abs(ratio - b["approx_ratio"]) < 0.04
    c = g["gpt3_mha_cache"]
    e = O.mha_kv_elements_per_token(c["layers"], c["heads"], c["d_k"])
    assert e == 2359296 and abs(e - c["elements_per_token_approx"]) / e < 0.01
    assert abs(e * c["bytes_per_elem"] / 1e6 - c["mb_per_token_approx"]) < 0.05
    gb = e * c["bytes_per_elem"] * c["context_tokens"] / 1e9
    assert abs(gb - c["gb_at_context_approx"]) / gb < 0.05
    d = g["qk_head_dim"]
    assert d["d_nope"] + d["d_rope"] == d["qk_dims"]
    h = g["head_dims_compute"]
    assert h["head_dims_big"] // h["head_dims_small"] == h["ratio"]


def test_cache_layout_bytes_per_token():
    assert O.kv_bytes_per_token(64, 16, "f32") == 320
    assert O.kv_bytes_per_token(512, 64, "bf16") == 1152
    assert O.kv_bytes_per_token(512, 64, "fp8") == 512 + 4 + 128 == 644
    assert O.block_bytes(64, 512, 64, "fp8") == 41216


# ---------------------------------------------------------------- append pins

@pytest.mark.parametrize("cache_dtype", ["f32", "bf16", "fp8"])
def test_append_layout_roundtrip(cache_dtype):
    """Write tokens with the layout writer, read them back through the block table
    with torch indexing (a different route), and check untouched bytes stay poisoned."""
    r = _rng(70)
    bs, d_c, d_R = 8, 16, 4
    seqlens = torch.tensor([13, 1, 20], dtype=torch.int32)
    table, n_phys = S.make_block_table(seqlens, bs, True, torch.Generator().manual_seed(3), 2)
    T = int(seqlens.sum())
    c = torch.from_numpy(r.standard_normal((T, d_c)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    kr = torch.from_numpy(r.standard_normal((T, d_R)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    seq = np.repeat(np.arange(3), seqlens.numpy())
    pos = np.concatenate([np.arange(L) for L in seqlens.tolist()])
    bb = O.block_bytes(bs, d_c, d_R, cache_dtype)
    poison = np.full(n_phys * bb, 0xA5, dtype=np.uint8)
    pool = O.append_expected_pool(poison, c, kr, seq, pos, table.numpy(), block_size=bs, d_c=d_c,
                                  d_rope=d_R, cache_dtype=cache_dtype, base=10000.0)
    tp = torch.from_numpy(pool).view(n_phys, bb)
    touched = torch.zeros(n_phys, bs, dtype=torch.bool)
    for n in range(T):
        blk = int(table[seq[n], pos[n] // bs]); slot = pos[n] % bs
        touched[blk, slot] = True
        want_c, want_k = O.cached_token_values(c[n:n + 1], kr[n:n + 1], pos[n:n + 1], cache_dtype, 10000.0)
        if cache_dtype == "f32":
            row = tp[blk, slot * (d_c + d_R) * 4:(slot + 1) * (d_c + d_R) * 4].view(torch.float32).double().numpy()
            got_c, got_k = row[:d_c], row[d_c:]
        elif cache_dtype == "bf16":
            row = tp[blk, slot * (d_c + d_R) * 2:(slot + 1) * (d_c + d_R) * 2].view(torch.bfloat16).double().numpy()
            got_c, got_k = row[:d_c], row[d_c:]
        else:
            codes = tp[blk, slot * d_c:(slot + 1) * d_c].view(torch.float8_e4m3fn).double().numpy()
            sc = tp[blk, bs * d_c + slot * 4: bs * d_c + slot * 4 + 4].view(torch.float32).double().numpy()
            got_c = codes * sc[0]
            off = bs * d_c + bs * 4 + slot * d_R * 2
            got_k = tp[blk, off:off + d_R * 2].view(torch.bfloat16).double().numpy()
        assert np.array_equal(got_c, want_c[0]) and np.array_equal(got_k, want_k[0])
    # every byte of an untouched slot (and of spare blocks) keeps the poison
    for blk in range(n_phys):
        for slot in range(bs):
            if touched[blk, slot]:
                continue
            if cache_dtype == "fp8":
                spans = [(slot * d_c, d_c), (bs * d_c + slot * 4, 4), (bs * d_c + bs * 4 + slot * d_R * 2, d_R * 2)]
            else:
                w = (d_c + d_R) * (4 if cache_dtype == "f32" else 2)
                spans = [(slot * w, w)]
            for off, n in spans:
                assert bool((tp[blk, off:off + n] == 0xA5).all())


def test_generator_block_table_and_positions():
    w = S.WORKLOADS["ragged_sq2"].replace(batch=5, seqlen_range=(3, 200))
    inp = S.make_inputs(w, 7)
    L = inp["seqlens"]
    assert int(L.min()) >= 2
    # every referenced physical block is distinct; padding is -1
    t = inp["block_table"]
    used = t[t >= 0]
    assert used.numel() == len(set(used.tolist()))
    nb = (L + 63) // 64
    for b in range(5):
        assert bool((t[b, :nb[b]] >= 0).all()) and bool((t[b, nb[b]:] == -1).all())
    assert torch.equal(inp["tok_pos"][inp["cu_seqlens"][1]:inp["cu_seqlens"][2]], torch.arange(int(L[1]), dtype=torch.int32))


# ---------------------------------------------------------------- prefill (MHA form) pins

def _prefill_problem(seed, T, H=3, d_c=16, d_nope=8, d_rope=4, d_v=6):
    r = _rng(seed)
    return dict(q_nope=r.standard_normal((T, H, d_nope)), q_rope=r.standard_normal((T, H, d_rope)),
                c=r.standard_normal((T, d_c)), kr=r.standard_normal((T, d_rope)),
                w_uk=r.standard_normal((H, d_nope, d_c)) / 4, w_uv=r.standard_normal((H, d_v, d_c)) / 4,
                scale=1 / math.sqrt(d_nope + d_rope), base=10000.0)


def test_prefill_single_token_returns_its_value():
    P = _prefill_problem(70, T=1)
    o, lse = O.prefill_mha_form(P["q_nope"], P["q_rope"], P["c"], P["kr"], P["w_uk"], P["w_uv"], P["scale"],
                                P["base"])
    for s in range(3):
        assert np.allclose(o[0, s], P["w_uv"][s] @ P["c"][0], rtol=1e-13)
    # one key: lse is that key's scaled score
    z0 = [P["scale"] * np.dot(np.concatenate([P["q_nope"][0, s], O.rope(P["q_rope"][0:1, s], np.array([0]),
                                                                          P["base"])[0]]),
                              np.concatenate([P["w_uk"][s] @ P["c"][0],
                                              O.store_value(O.rope(P["kr"][0:1], np.array([0]), P["base"]), "bf16")[0]]))
          for s in range(3)]
    assert np.allclose(lse[0], z0, rtol=1e-12)


def test_prefill_matches_torch_causal_sdpa():
    """Against torch's causal scaled-dot-product attention (float64, CPU) on the
    explicitly decompressed per-head keys and values."""
    P = _prefill_problem(71, T=37)
    T = 37
    o, lse = O.prefill_mha_form(P["q_nope"], P["q_rope"], P["c"], P["kr"], P["w_uk"], P["w_uv"], P["scale"],
                                P["base"])
    pos = np.arange(T)
    qr = O.rope(P["q_rope"], pos[:, None], P["base"])
    kr = O.store_value(O.rope(P["kr"], pos, P["base"]), "bf16")
    for s in range(3):
        q = torch.from_numpy(np.concatenate([P["q_nope"][:, s], qr[:, s]], axis=1))[None, None]
        k = torch.from_numpy(np.concatenate([P["c"] @ P["w_uk"][s].T, kr], axis=1))[None, None]
        v = torch.from_numpy(P["c"] @ P["w_uv"][s].T)[None, None]
        want = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=P["scale"])
        assert np.allclose(o[:, s], want[0, 0].numpy(), rtol=1e-11, atol=1e-12)


def test_prefill_rows_are_decodes_of_their_prefix():
    """Row i of a prefill equals decoding the first i+1 tokens with one query
    at position i (the decode oracle, pinned above, on a bf16-stored k_R)."""
    P = _prefill_problem(72, T=19)
    o, lse = O.prefill_mha_form(P["q_nope"], P["q_rope"], P["c"], P["kr"], P["w_uk"], P["w_uv"], P["scale"],
                                P["base"])
    for i in [0, 1, 7, 18]:
        kr_c = O.store_value(O.rope(P["kr"][:i + 1], np.arange(i + 1), P["base"]), "bf16")
        od, _, ld = O.decode_mha_form(P["q_nope"][i:i + 1], P["q_rope"][i:i + 1], P["c"][:i + 1], kr_c,
                                      np.array([i]), P["w_uk"], P["w_uv"], P["scale"], P["base"])
        assert np.allclose(o[i], od[0], rtol=1e-12, atol=1e-13)
        assert np.allclose(lse[i], ld[0], rtol=1e-12)


def test_prefill_is_causal():
    """Changing tokens after row i leaves rows 0..i unchanged."""
    P = _prefill_problem(73, T=16)
    o1, _ = O.prefill_mha_form(P["q_nope"], P["q_rope"], P["c"], P["kr"], P["w_uk"], P["w_uv"], P["scale"],
                               P["base"])
    P2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in P.items()}
    P2["c"][9:] += 5.0
    P2["kr"][9:] -= 3.0
    P2["q_nope"][9:] *= 2.0
    o2, _ = O.prefill_mha_form(P2["q_nope"], P2["q_rope"], P2["c"], P2["kr"], P2["w_uk"], P2["w_uv"], P2["scale"],
                               P2["base"])
    assert np.array_equal(o1[:9], o2[:9])
    assert not np.allclose(o1[9:], o2[9:])


def test_prefill_chunk_rows_equal_whole_prompt_rows():
    """A chunk of the last Lq tokens attending to the whole prompt gives the
    last Lq rows of the whole prompt's prefill, for every split point."""
    P = _prefill_problem(75, T=23)
    o, lse = O.prefill_mha_form(P["q_nope"], P["q_rope"], P["c"], P["kr"], P["w_uk"], P["w_uv"], P["scale"],
                                P["base"])
    kr_c = O.store_value(O.rope(P["kr"], np.arange(23), P["base"]), "bf16")
    for lq in [1, 5, 22, 23]:
        oc, lc = O.prefill_chunk_mha_form(P["q_nope"][23 - lq:], P["q_rope"][23 - lq:], P["c"], kr_c, P["w_uk"],
                                          P["w_uv"], P["scale"], P["base"])
        assert np.allclose(oc, o[23 - lq:], rtol=1e-12, atol=1e-13)
        assert np.allclose(lc, lse[23 - lq:], rtol=1e-12)
    # a chunk's rows do not depend on tokens after the chunk's own positions
    oc2, _ = O.prefill_chunk_mha_form(P["q_nope"][10:12], P["q_rope"][10:12], P["c"][:12], kr_c[:12], P["w_uk"],
                                      P["w_uv"], P["scale"], P["base"])
    assert np.allclose(oc2, o[10:12], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- output gate (gated MLA)

def test_output_gate_closed_forms():
    r = _rng(21)
    o = r.standard_normal((3, 4, 8))
    # sigma(0) = 1/2 and sigma(ln 3) = 3/4 exactly (e^-ln3 = 1/3)
    assert np.allclose(O.output_gate(o, np.zeros_like(o)), o / 2, rtol=0, atol=1e-15)
    assert np.allclose(O.output_gate(o, np.full_like(o, math.log(3.0))), 0.75 * o, rtol=1e-15, atol=1e-15)
    # saturation without overflow: a large positive logit passes o, a large negative one closes the gate
    with np.errstate(over="raise", invalid="raise", divide="raise"):
        assert np.array_equal(O.output_gate(o, np.full_like(o, 800.0)), o)
        assert np.array_equal(O.output_gate(o, np.full_like(o, -800.0)), np.zeros_like(o))


def test_output_gate_symmetry_and_library_logistic():
    from scipy.special import expit
    r = _rng(22)
    o = r.standard_normal((5, 3, 16))
    g = r.standard_normal((5, 3, 16)) * 6
    # sigma(g) + sigma(-g) = 1, so the two gated outputs add up to the ungated one
    assert np.allclose(O.output_gate(o, g) + O.output_gate(o, -g), o, rtol=0, atol=1e-14)
    # the logistic function of scipy
    assert np.allclose(O.output_gate(o, g), o * expit(g), rtol=1e-14, atol=1e-15)
    # the gate only shrinks: |out| <= |o| elementwise, with the sign of o
    out = O.output_gate(o, g)
    assert np.all(np.abs(out) <= np.abs(o)) and np.all(out * o >= 0)


# ---------------------------------------------------------------- upstream projections

def test_project_down_selection_rows_copy_coordinates():
    """Unit-vector rows of W_down pick coordinates of h: the projections are
    those coordinates, exact whenever they are bf16 values already."""
    r = _rng(31)
    d_model, d_cq, d_c, d_r = 40, 6, 8, 4
    h = O.to_bf16_value(r.standard_normal((5, d_model)))
    pick = r.permutation(d_model)[:d_cq + d_c + d_r]
    W = np.zeros((d_cq + d_c + d_r, d_model))
    W[np.arange(len(pick)), pick] = 1.0
    cq, ckv, kr = O.project_down(h, W, d_cq, d_c, d_r)
    assert np.array_equal(np.concatenate([cq, ckv, kr], axis=1), h[:, pick])


def test_project_down_brute_force_and_rounding():
    r = _rng(32)
    h, W = r.standard_normal((3, 10)), r.standard_normal((7, 10))
    cq, ckv, kr = O.project_down(h, W, 2, 3, 2, out_dtype=None)
    y = np.concatenate([cq, ckv, kr], axis=1)
    for t in range(3):
        for n in range(7):
            assert abs(y[t, n] - sum(h[t, k] * W[n, k] for k in range(10))) < 1e-12
    yb = np.concatenate(O.project_down(h, W, 2, 3, 2), axis=1)
    # one rounding to bf16 (8 significant bits): within half an ulp, at most 2^-8 relative, and on the bf16 grid
    assert np.all(np.abs(yb - y) <= np.abs(y) * 2.0 ** -8)
    assert np.array_equal(O.to_bf16_value(yb), yb)


def test_query_from_latent_equals_the_composed_absorbed_map():
    """Without the intermediate rounding, W_UK^T (W_UQ c) is the composed map
    (W_UK^T W_UQ) c: the absorption of W_UK into the query projection
    ([P4] 为什么需要解耦 RoPE; [P1] 双重投影, q = x W_q W_k^T)."""
    r = _rng(33)
    H, d_nope, d_r, d_c, d_cq, n = 3, 8, 4, 16, 12, 5
    c_q = r.standard_normal((n, d_cq))
    w_uq = r.standard_normal((H, d_nope + d_r, d_cq))
    w_uk = r.standard_normal((H, d_nope, d_c))
    pos = np.array([0, 1, 5, 100, 7])
    qa = O.query_from_latent(c_q, w_uq, pos, w_uk, d_nope, 10000.0, out_dtype=None)
    for s in range(H):
        composed = w_uk[s].T @ w_uq[s, :d_nope]                  # [d_c, d_cq]
        assert np.allclose(qa[:, s, :d_c], c_q @ composed.T, rtol=1e-12, atol=1e-12)
        # the RoPE part is the rotated W_QR c_Q
        qr = c_q @ w_uq[s, d_nope:].T
        assert np.allclose(qa[:, s, d_c:], O.rope(qr, pos, 10000.0), rtol=1e-12, atol=1e-12)
    # with the bf16 reading, the intermediate is on the bf16 grid and the result moves by about its resolution
    qb = O.query_from_latent(c_q, w_uq, pos, w_uk, d_nope, 10000.0)
    rel = np.linalg.norm(qb - qa) / np.linalg.norm(qa)
    assert 1e-5 < rel < 1e-2
