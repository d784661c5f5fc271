"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own code path: a hand-derived
worked example, brute force with scalar loops, closed forms, an algebraically
different (absorbed) evaluation, library scaled-dot-product attention, torch's
float8_e4m3fn casts, and RoPE's defining properties.  A plausible mistake in
the oracle (a dropped term, a wrong sign, scale or index, a transposed
operand, an off-by-one causal extent) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats, mla
from oracle.rope import rope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _expr(v):
    """Evaluate the tiny log expressions used in the golden file."""
    if isinstance(v, (int, float)):
        return float(v)
    env = {"ln2": math.log(2), "ln3": math.log(3), "ln5": math.log(5),
           "ln9": math.log(9), "ln10": math.log(10)}
    return float(eval(v, {"__builtins__": {}}, env))


def _golden():
    with open(os.path.join(GOLDEN, "mla_worked_example.json")) as f:
        return json.load(f)


def _golden_operands(g):
    d = g["dims"]
    H, dh, dc = d["n_heads"], d["d_head"], d["d_latent"]
    w_uk = np.array(g["w_uk_full"], dtype=np.float64).reshape(H, dh, dc)
    w_uv = np.array(g["w_uv_full"], dtype=np.float64).reshape(H, dh, dc)
    C = np.array(g["cache"]["c_kv"], dtype=np.float64)
    KR = np.array(g["cache"]["k_r"], dtype=np.float64)
    qn = np.array([[_expr(x) for x in row] for row in g["query"]["q_nope"]])
    qr = np.array([[_expr(x) for x in row] for row in g["query"]["q_rope"]])
    return w_uk, w_uv, C, KR, qn, qr


# ---------------------------------------------------------------- worked example
def test_golden_worked_example_T1():
    g = _golden()
    w_uk, w_uv, C, KR, qn, qr = _golden_operands(g)
    out = mla.decode(qn[None], qr[None], w_uk, w_uv, C, KR,
                     np.array([0, 2]), np.array([2]), q_tokens=1)
    e = g["expected_T1"]
    np.testing.assert_allclose(out["o"][0], e["o"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(out["latent"][0], e["latent"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(out["lse"][0], [_expr(x) for x in e["lse"]],
                               rtol=0, atol=1e-13)


def test_golden_worked_example_T2_causal():
    g = _golden()
    w_uk, w_uv, C, KR, qn, qr = _golden_operands(g)
    qn2 = np.stack([qn, qn])
    qr2 = np.stack([qr, qr])
    out = mla.decode(qn2, qr2, w_uk, w_uv, C, KR, np.array([0, 2]),
                     np.array([2]), q_tokens=2)
    e0, e1 = g["expected_T2_tau0"], g["expected_T1"]
    np.testing.assert_allclose(out["o"][0], e0["o"], atol=1e-13)
    np.testing.assert_allclose(out["latent"][0], e0["latent"], atol=1e-13)
    np.testing.assert_allclose(out["lse"][0], [_expr(x) for x in e0["lse"]], atol=1e-13)
    np.testing.assert_allclose(out["o"][1], e1["o"], atol=1e-13)
    np.testing.assert_allclose(out["lse"][1], [_expr(x) for x in e1["lse"]], atol=1e-13)


# ------------------------------------------------------------------ brute force
def _brute_force(q_nope, q_rope, W_UK_full, W_UV_full, C, KR, L, T, d_h):
    """Scalar loops straight from the equations (tiny sizes only).

    W_*_full are the [d_h n_h x d_c] matrices; head i uses rows i*d_h + r.
    """
    n_h = len(q_nope[0])
    d_c = len(C[0])
    d_r = len(KR[0])
    res = {}
    for tau in range(T):
        t = L - T + tau                    # 0-based position of the query
        for i in range(n_h):
            scores = []
            for j in range(t + 1):
                acc = 0.0
                for r in range(d_h):
                    kc = sum(W_UK_full[i * d_h + r][c] * C[j][c] for c in range(d_c))
                    acc += q_nope[tau][i][r] * kc
                for r in range(d_r):
                    acc += q_rope[tau][i][r] * KR[j][r]
                scores.append(acc / math.sqrt(d_h + d_r))
            mx = max(scores)
            ex = [math.exp(s - mx) for s in scores]
            z = sum(ex)
            o = []
            for r in range(d_h):
                o.append(sum(ex[j] / z * sum(W_UV_full[i * d_h + r][c] * C[j][c]
                                             for c in range(d_c))
                             for j in range(t + 1)))
            res[(tau, i)] = (o, mx + math.log(z))
    return res


@pytest.mark.parametrize("T", [1, 2, 3])
def test_brute_force_tiny(T):
    rng = np.random.default_rng(1234 + T)
    n_h, d_h, d_c, d_r, L = 2, 3, 4, 2, 3
    W_UK_full = rng.standard_normal((n_h * d_h, d_c))
    W_UV_full = rng.standard_normal((n_h * d_h, d_c))
    C = rng.standard_normal((L, d_c))
    KR = rng.standard_normal((L, d_r))
    qn = rng.standard_normal((T, n_h, d_h))
    qr = rng.standard_normal((T, n_h, d_r))
    out = mla.decode(qn, qr, W_UK_full.reshape(n_h, d_h, d_c),
                     W_UV_full.reshape(n_h, d_h, d_c), C, KR,
                     np.array([0, L]), np.array([L]), q_tokens=T)
    bf = _brute_force(qn.tolist(), qr.tolist(), W_UK_full.tolist(),
                      W_UV_full.tolist(), C.tolist(), KR.tolist(), L, T, d_h)
    for (tau, i), (o, lse) in bf.items():
        np.testing.assert_allclose(out["o"][tau, i], o, rtol=1e-12, atol=1e-12)
        assert abs(out["lse"][tau, i] - lse) < 1e-12


# ------------------------------------------------------------------ closed forms
def _rand_problem(rng, n_h=3, d_h=5, d_c=7, d_r=4, L=6, T=1):
    return dict(
        w_uk=rng.standard_normal((n_h, d_h, d_c)) / math.sqrt(d_c),
        w_uv=rng.standard_normal((n_h, d_h, d_c)) / math.sqrt(d_c),
        C=rng.standard_normal((L, d_c)), KR=rng.standard_normal((L, d_r)),
        qn=rng.standard_normal((T, n_h, d_h)), qr=rng.standard_normal((T, n_h, d_r)),
        L=L, T=T)


def _run(p, **kw):
    return mla.decode(p["qn"], p["qr"], p["w_uk"], p["w_uv"], p["C"], p["KR"],
                      np.array([0, p["L"]]), np.array([p["L"]]), p["T"], **kw)


def test_closed_form_single_token():
    """L = 1: softmax over one key is 1, so o = W^UV_i c_0 and latent = c_0."""
    p = _rand_problem(np.random.default_rng(5), L=1)
    out = _run(p)
    for i in range(p["w_uk"].shape[0]):
        np.testing.assert_allclose(out["o"][0, i], p["w_uv"][i] @ p["C"][0], rtol=1e-14)
        np.testing.assert_allclose(out["latent"][0, i], p["C"][0], rtol=1e-14)


def test_closed_form_uniform_softmax():
    """q = 0: every score is 0, p is uniform, LSE = ln L, o = W^UV_i mean(c)."""
    p = _rand_problem(np.random.default_rng(6), L=9)
    p["qn"][:] = 0
    p["qr"][:] = 0
    out = _run(p)
    mean_c = p["C"].mean(axis=0)
    for i in range(p["w_uk"].shape[0]):
        np.testing.assert_allclose(out["o"][0, i], p["w_uv"][i] @ mean_c, rtol=1e-13)
        np.testing.assert_allclose(out["latent"][0, i], mean_c, rtol=1e-13)
        assert abs(out["lse"][0, i] - math.log(9)) < 1e-14


def test_softmax_weights_sum_to_one():
    """With W^UK = 0 the scores come from the RoPE part only; with all-ones
    latent rows, latent = sum_j p_j * 1 must be exactly 1 for any scores."""
    rng = np.random.default_rng(7)
    p = _rand_problem(rng, L=11)
    p["w_uk"][:] = 0
    p["C"][:] = 1.0
    p["qr"] *= 3.0
    out = _run(p)
    np.testing.assert_allclose(out["latent"], 1.0, rtol=0, atol=1e-14)


def test_scale_is_pre_absorption_head_dim():
    """Scaling q by a changes the scores by a; the scale must be
    1/sqrt(d_h + d_h^R) (not 1/sqrt(d_c)): with L = 2 and one nonzero score
    s_1 = x * scale, the LSE is ln(1 + e^{s_1})."""
    n_h, d_h, d_c, d_r = 1, 3, 8, 2
    w_uk = np.zeros((1, d_h, d_c)); w_uk[0, 0, 0] = 1.0
    w_uv = np.zeros((1, d_h, d_c))
    C = np.zeros((2, d_c)); C[1, 0] = 1.0
    KR = np.zeros((2, d_r))
    qn = np.zeros((1, 1, d_h)); qn[0, 0, 0] = 2.0
    qr = np.zeros((1, 1, d_r))
    out = mla.decode(qn, qr, w_uk, w_uv, C, KR, np.array([0, 2]), np.array([2]), 1)
    s1 = 2.0 / math.sqrt(d_h + d_r)
    assert abs(out["lse"][0, 0] - math.log(1 + math.exp(s1))) < 1e-14


# ---- absorption identity ("DeepSeek-V2: Strong, Economical, Efficient", 2.1.2, App. C)
def _absorbed(p):
    """Absorbed evaluation (DeepSeek-V2 Appendix C: W^UK folded into the query,
    W^UV applied after the latent-space sum), written independently."""
    n_h, d_h, d_c = p["w_uk"].shape
    d_r = p["KR"].shape[1]
    L, T = p["L"], p["T"]
    o = np.zeros((T, n_h, d_h)); lat = np.zeros((T, n_h, d_c)); lse = np.zeros((T, n_h))
    cache = np.concatenate([p["C"], p["KR"]], axis=1)
    for tau in range(T):
        n = L - T + tau + 1
        for i in range(n_h):
            q_abs = np.concatenate([p["w_uk"][i].T @ p["qn"][tau, i], p["qr"][tau, i]])
            s = cache[:n] @ q_abs / math.sqrt(d_h + d_r)
            m = s.max()
            w = np.exp(s - m)
            lat[tau, i] = (w @ p["C"][:n]) / w.sum()
            o[tau, i] = p["w_uv"][i] @ lat[tau, i]
            lse[tau, i] = m + math.log(w.sum())
    return o, lat, lse


@pytest.mark.parametrize("T", [1, 4])
def test_absorbed_identity(T):
    p = _rand_problem(np.random.default_rng(11 + T), n_h=4, d_h=8, d_c=16, d_r=4,
                      L=37, T=T)
    out = _run(p)
    o, lat, lse = _absorbed(p)
    for a, b in ((out["o"], o), (out["latent"], lat), (out["lse"], lse)):
        assert np.linalg.norm(a - b) <= 1e-12 * np.linalg.norm(b)


def test_rope_on_compressed_key_breaks_absorption():
    """Decoupled-RoPE rationale (DeepSeek-V2 section 2.1.3): rotating k^C by a
    position-dependent RoPE leaves no position-independent absorbed query,
    while rotating only k^R keeps the identity."""
    rng = np.random.default_rng(3)
    d_h, d_c, L = 4, 6, 5
    W = rng.standard_normal((d_h, d_c))
    C = rng.standard_normal((L, d_c))
    qc = rng.standard_normal(d_h)
    pos = np.arange(L)
    q_abs = W.T @ qc
    plain = (C @ W.T) @ qc
    absorbed = C @ q_abs
    rotated = np.array([rope((W @ C[j])[None], pos[j:j + 1])[0] @ qc for j in range(L)])
    assert np.allclose(plain, absorbed, rtol=1e-13)
    assert not np.allclose(rotated, absorbed, rtol=1e-3)


# ------------------------------------------------ library attention (SDPA), fp64
@pytest.mark.parametrize("T", [1, 3])
def test_matches_library_sdpa(T):
    rng = np.random.default_rng(21 + T)
    n_h, d_h, d_c, d_r, L = 3, 8, 12, 4, 29
    p = _rand_problem(rng, n_h=n_h, d_h=d_h, d_c=d_c, d_r=d_r, L=L, T=T)
    out = _run(p)
    C = torch.from_numpy(p["C"])
    KR = torch.from_numpy(p["KR"])
    scale = 1.0 / math.sqrt(d_h + d_r)
    # causal mask: query tau sees positions 0 .. L - T + tau
    mask = torch.arange(L)[None, :] <= (L - T + torch.arange(T))[:, None]
    for i in range(n_h):
        K = torch.cat([C @ torch.from_numpy(p["w_uk"][i]).T, KR], dim=1)
        V = C @ torch.from_numpy(p["w_uv"][i]).T
        q = torch.cat([torch.from_numpy(p["qn"][:, i]), torch.from_numpy(p["qr"][:, i])], 1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[None, None], K[None, None], V[None, None], attn_mask=mask[None, None],
            scale=scale)[0, 0].numpy()
        np.testing.assert_allclose(out["o"][:, i], ref, rtol=1e-12, atol=1e-13)
        # absorbed form = MQA over the cache rows, value = latent row
        q_abs = torch.cat([torch.from_numpy(p["qn"][:, i]) @ torch.from_numpy(p["w_uk"][i]),
                           torch.from_numpy(p["qr"][:, i])], 1)
        lat = torch.nn.functional.scaled_dot_product_attention(
            q_abs[None, None], torch.cat([C, KR], 1)[None, None], C[None, None],
            attn_mask=mask[None, None], scale=scale)[0, 0].numpy()
        np.testing.assert_allclose(out["latent"][:, i], lat, rtol=1e-12, atol=1e-13)


# -------------------------------------------------------- split / LSE combine
def test_split_then_lse_combine_equals_whole():
    rng = np.random.default_rng(8)
    d_h, d_c, d_r, L = 4, 8, 2, 50
    w_uk = rng.standard_normal((d_h, d_c)); w_uv = rng.standard_normal((d_h, d_c))
    C = rng.standard_normal((L, d_c)) * 2; KR = rng.standard_normal((L, d_r))
    qc = rng.standard_normal(d_h); qr = rng.standard_normal(d_r)
    scale = 1 / math.sqrt(d_h + d_r)
    o, lat, lse = mla.attend_head(qc, qr, C, KR, w_uk, w_uv, scale)
    cuts = [0, 7, 8, 31, 50]
    parts = [mla.attend_head(qc, qr, C[a:b], KR[a:b], w_uk, w_uv, scale)
             for a, b in zip(cuts[:-1], cuts[1:])]
    lses = np.array([x[2] for x in parts])
    tot = np.logaddexp.reduce(lses)
    wts = np.exp(lses - tot)
    assert abs(tot - lse) < 1e-12
    np.testing.assert_allclose(sum(w * x[0] for w, x in zip(wts, parts)), o, rtol=1e-12)
    np.testing.assert_allclose(sum(w * x[1] for w, x in zip(wts, parts)), lat, rtol=1e-12)


def test_causal_T4_equals_T1_on_truncated_cache():
    rng = np.random.default_rng(9)
    p = _rand_problem(rng, n_h=2, d_h=4, d_c=6, d_r=2, L=20, T=4)
    out = _run(p)
    for tau in range(4):
        Lt = 20 - 4 + tau + 1
        q = dict(p, C=p["C"][:Lt], KR=p["KR"][:Lt], qn=p["qn"][tau:tau + 1],
                 qr=p["qr"][tau:tau + 1], L=Lt, T=1)
        one = _run(q)
        np.testing.assert_allclose(out["o"][tau], one["o"][0], rtol=1e-13)
        np.testing.assert_allclose(out["lse"][tau], one["lse"][0], rtol=1e-13)


# ----------------------------------------------------------------- FP8 E4M3
def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = formats.E4M3_TABLE
    assert np.array_equal(np.isnan(ref), np.isnan(tab))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], tab[ok])


def test_e4m3_format_landmarks():
    # OCP E4M3: max 448, min normal 2^-6, min subnormal 2^-9, NaN = S.1111.111
    assert formats.E4M3_TABLE[0x7E] == 448.0
    assert formats.E4M3_TABLE[0x08] == 2.0 ** -6
    assert formats.E4M3_TABLE[0x01] == 2.0 ** -9
    assert np.isnan(formats.E4M3_TABLE[0x7F]) and np.isnan(formats.E4M3_TABLE[0xFF])
    assert np.isfinite(formats.E4M3_TABLE[0x78])  # e=15 is not reserved for inf


def test_e4m3_rounding_matches_torch_cast():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 60,
        rng.standard_normal(20000).astype(np.float32) * 1e-2,
        # exact midpoints between neighbouring codes (ties -> even)
        ((formats.E4M3_TABLE[1:0x7E] + formats.E4M3_TABLE[2:0x7F]) / 2).astype(np.float32),
        -((formats.E4M3_TABLE[0:0x7D] + formats.E4M3_TABLE[1:0x7E]) / 2).astype(np.float32),
        np.array([0.0, 448.0, -448.0, 447.9, 464.0, 2.0 ** -10], dtype=np.float32),
    ])
    vals = np.clip(vals, -448.0, 448.0).astype(np.float32)
    ours = formats.f32_to_e4m3_rne_sat(vals)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates_above_max():
    v = np.array([449.0, 470.0, 1e6, -1e6], dtype=np.float32)
    assert np.all(formats.e4m3_to_f64(formats.f32_to_e4m3_rne_sat(v)) ==
                  np.array([448.0, 448.0, 448.0, -448.0]))


def test_per_token_quantisation_bounds():
    rng = np.random.default_rng(2)
    rows = rng.standard_normal((300, 576)).astype(np.float32)
    rows[0] = 0.0
    rows[1] *= 1e-30
    codes, scales = formats.quantize_rows_e4m3(rows)
    assert scales[0] == 1.0 and np.all(codes[0] & 0x7F == 0)
    deq = formats.dequantize_rows_e4m3(codes, scales)
    mags = np.abs(formats.e4m3_to_f64(codes[1:]))
    assert np.all(mags.max(axis=1) == 448.0)            # amax maps to 448
    # error of nearest rounding: half a code step, relative 2^-4 (normals),
    # absolute 2^-10 * s (subnormals)
    err = np.abs(deq - rows.astype(np.float64))
    bound = np.maximum(np.abs(rows) * 2.0 ** -4, 2.0 ** -10 * scales[:, None]) * (1 + 1e-6)
    assert np.all(err <= bound)


# ---------------------------------------------------------------------- RoPE
def test_rope_identity_at_zero_and_known_angle():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 16))
    np.testing.assert_array_equal(rope(x, np.zeros(5)), x)
    # d = 2: theta_0 = 1, position 1 rotates by 1 radian
    y = rope(np.array([[1.0, 0.0]]), np.array([1]))
    np.testing.assert_allclose(y[0], [math.cos(1.0), math.sin(1.0)], rtol=1e-15)
    # d = 4, base 100: theta_1 = 100^(-1/2) = 0.1
    y = rope(np.array([[0.0, 0.0, 1.0, 0.0]]), np.array([10]), base=100.0)
    np.testing.assert_allclose(y[0, 2:], [math.cos(1.0), math.sin(1.0)], rtol=1e-14)


def test_rope_relative_position_property():
    rng = np.random.default_rng(5)
    x, y = rng.standard_normal(64), rng.standard_normal(64)
    for m, n, k in [(5, 2, 2), (100, 7, 50), (63, 0, 63)]:
        a = rope(x[None], np.array([m]))[0] @ rope(y[None], np.array([n]))[0]
        b = rope(x[None], np.array([m - k]))[0] @ rope(y[None], np.array([n - k]))[0]
        assert abs(a - b) < 1e-10
    np.testing.assert_allclose(np.linalg.norm(rope(x[None], np.array([77]))), np.linalg.norm(x))


# ---------------------------------------------------------- cache accounting
def test_kv_cache_accounting_matches_pages():
    with open(os.path.join(GOLDEN, "kv_cache_per_token.json")) as f:
        g = json.load(f)
    v2 = g["deepseek_v2"]
    from mla_inputs import WORKLOADS
    w = WORKLOADS["v2_b32_l4k_bf16"]
    assert (w.n_heads, w.d_head, w.d_latent, w.d_rope) == (
        v2["n_h"], v2["d_h"], v2["d_c"], v2["d_h_rope"])
    e = g["expected"]
    mha = 2 * w.n_heads * w.d_head
    mla_el = w.d_latent + w.d_rope
    assert mha == e["mha_elements"] and mla_el == e["mla_elements"]
    assert w.d_latent == 4 * w.d_head and w.d_rope == w.d_head // 2
    assert mla_el / w.d_head == e["mla_over_d_h"]
    assert mla_el / (2 * w.d_head) == e["gqa_equivalent_groups"]
    assert 2 * mla_el == e["bf16_bytes_per_token"]
    assert mla_el + 4 == e["fp8_bytes_per_token_with_fp32_scale"]


def test_cache_row_index_hand_computed_slots():
    """The slot map of the cache layouts, against slots worked out by hand.

    Paged, 4-token pages, two sequences with shuffled pages: sequence 0 owns
    pages [2, 0] (tokens 0-3 -> rows 8-11, tokens 4-7 -> rows 0-3), sequence 1
    owns pages [1, 3] (tokens 0-3 -> rows 4-7, tokens 4-7 -> rows 12-15).
    Contiguous with max_len 10: row = 10 * seq + pos."""
    pt = np.array([[2, 0], [1, 3]])
    seq = np.array([0, 0, 0, 1, 1, 1, 1])
    pos = np.array([0, 3, 5, 0, 3, 4, 7])
    assert mla.cache_row_index(seq, pos, pt, 4, 0).tolist() == [8, 11, 1, 4, 7, 12, 15]
    assert mla.cache_row_index(seq, pos, None, 4, 10).tolist() == [0, 3, 5, 10, 13, 14, 17]
    # 64-token pages: token 130 of a sequence with pages [5, 1, 3] is entry 2
    # of page 3 (130 = 2 * 64 + 2) -> row 3 * 64 + 2 = 194; token 63 -> row 383
    pt64 = np.array([[5, 1, 3]])
    assert mla.cache_row_index(np.array([0, 0, 0]), np.array([130, 63, 64]), pt64, 64,
                               0).tolist() == [194, 383, 64]
    # every (sequence, position) of a full table lands on its own slot
    all_seq = np.repeat([0, 1], 8)
    all_pos = np.tile(np.arange(8), 2)
    slots = mla.cache_row_index(all_seq, all_pos, pt, 4, 0)
    assert sorted(slots.tolist()) == list(range(16))


# ------------------------------------------- absorbed query and up-projection
def test_absorbed_query_reproduces_unabsorbed_scores():
    """q~ . [c_j ; k^R_j] must equal q . k_j with k_j = [W^UK_i c_j ; k^R_j]
    materialised from the definition."""
    rng = np.random.default_rng(31)
    n_h, d_h, d_c, d_r, L, N = 3, 6, 10, 4, 7, 2
    w_uk = rng.standard_normal((n_h, d_h, d_c))
    qn = rng.standard_normal((N, n_h, d_h)); qr = rng.standard_normal((N, n_h, d_r))
    C = rng.standard_normal((L, d_c)); KR = rng.standard_normal((L, d_r))
    qa = mla.absorbed_query(qn, qr, w_uk)
    assert qa.shape == (N, n_h, d_c + d_r)
    for n in range(N):
        for i in range(n_h):
            direct = np.array([sum(qn[n, i, r] * sum(w_uk[i, r, c] * C[j, c] for c in range(d_c))
                                   for r in range(d_h)) + qr[n, i] @ KR[j] for j in range(L)])
            np.testing.assert_allclose(np.concatenate([C, KR], 1) @ qa[n, i], direct, rtol=1e-12)


def test_up_project_matches_literal_values():
    """W^UV applied to the oracle's latent output equals the literal o."""
    p = _rand_problem(np.random.default_rng(32), n_h=3, d_h=5, d_c=9, d_r=2, L=13, T=2)
    out = _run(p)
    np.testing.assert_allclose(mla.up_project(out["latent"], p["w_uv"]), out["o"], rtol=1e-12)
    # and against the worked example
    g = _golden()
    w_uk, w_uv, C, KR, qn, qr = _golden_operands(g)
    lat = np.array(g["expected_T1"]["latent"])[None]
    np.testing.assert_allclose(mla.up_project(lat, w_uv)[0], g["expected_T1"]["o"], atol=1e-13)


# ------------------------------------------------ output projection (W^O)
def test_output_projection_absorbs_w_uv():
    """[V2] section 2.1.2: W^UV can be absorbed into W^O.  Projecting the
    up-projected heads, W^O [W^UV_1 lat_1; ...], equals applying the merged
    per-head matrices (W^O_i W^UV_i) to the latent rows directly."""
    rng = np.random.default_rng(41)
    n_tok, H, d_h, d_c, d = 3, 4, 5, 7, 6
    lat = rng.standard_normal((n_tok, H, d_c))
    w_uv = rng.standard_normal((H, d_h, d_c))
    w_o = rng.standard_normal((d, H * d_h))
    u = mla.output_project(mla.up_project(lat, w_uv), w_o)
    merged = [w_o[:, i * d_h:(i + 1) * d_h] @ w_uv[i] for i in range(H)]   # [d, d_c] each
    u2 = sum(lat[:, i, :] @ merged[i].T for i in range(H))
    np.testing.assert_allclose(u, u2, rtol=1e-12, atol=1e-12)


def test_output_projection_special_cases():
    """Identity W^O returns the concatenated heads in head order; a W^O with
    one nonzero column block reads only that head; a permutation of the
    output rows permutes u; the map is linear."""
    rng = np.random.default_rng(42)
    n_tok, H, d_h = 2, 3, 4
    o = rng.standard_normal((n_tok, H, d_h))
    u = mla.output_project(o, np.eye(H * d_h))
    np.testing.assert_array_equal(u, o.reshape(n_tok, H * d_h))
    blk = np.zeros((5, H * d_h))
    E = rng.standard_normal((5, d_h))
    blk[:, 2 * d_h:3 * d_h] = E
    np.testing.assert_allclose(mla.output_project(o, blk), o[:, 2, :] @ E.T, rtol=1e-13)
    w_o = rng.standard_normal((7, H * d_h))
    perm = rng.permutation(7)
    np.testing.assert_allclose(mla.output_project(o, w_o[perm]), mla.output_project(o, w_o)[:, perm],
                               rtol=1e-13)
    o2 = rng.standard_normal(o.shape)
    np.testing.assert_allclose(mla.output_project(2.0 * o - 3.0 * o2, w_o),
                               2.0 * mla.output_project(o, w_o) - 3.0 * mla.output_project(o2, w_o),
                               rtol=1e-12, atol=1e-12)


# ------------------------------------------------ cache producer (W^DKV, W^KR)
def test_producer_rms_norm_closed_forms():
    """With unit gain and eps = 0 every c part has RMS exactly 1; scaling h by
    a > 0 leaves the normalised c unchanged and scales k by a; the gain
    multiplies elementwise; without a gain c is the plain projection."""
    rng = np.random.default_rng(51)
    n, d, d_c, d_r = 4, 9, 6, 4
    h = rng.standard_normal((n, d))
    w_dkv, w_kr = rng.standard_normal((d_c, d)), rng.standard_normal((d_r, d))
    rows = mla.produce_rows(h, w_dkv, w_kr, np.ones(d_c), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(rows[:, :d_c] ** 2, axis=1)), 1.0, rtol=1e-13)
    rows3 = mla.produce_rows(3.0 * h, w_dkv, w_kr, np.ones(d_c), 0.0)
    np.testing.assert_allclose(rows3[:, :d_c], rows[:, :d_c], rtol=1e-12)
    np.testing.assert_allclose(rows3[:, d_c:], 3.0 * rows[:, d_c:], rtol=1e-12)
    g = rng.standard_normal(d_c)
    np.testing.assert_allclose(mla.produce_rows(h, w_dkv, w_kr, g, 0.0)[:, :d_c],
                               rows[:, :d_c] * g[None, :], rtol=1e-12)
    plain = mla.produce_rows(h, w_dkv, w_kr, None, 0.0)
    np.testing.assert_allclose(plain[:, :d_c], h @ w_dkv.T, rtol=1e-13)
    # eps: c / sqrt(mean c^2 + eps) for a row of equal entries 2: 2 / sqrt(4 + 5) = 2/3
    one = mla.produce_rows(np.ones((1, 1)), np.full((d_c, 1), 2.0), np.zeros((d_r, 1)),
                           np.ones(d_c), 5.0)
    np.testing.assert_allclose(one[0, :d_c], 2.0 / 3.0, rtol=1e-14)


def test_producer_selection_weights_and_rope():
    """Unit-vector rows of W^DKV / W^KR pick entries of h (catches a
    transposed operand); the k part is rotated at its token's position, and
    position 0 leaves it unrotated (R_0 = I)."""
    rng = np.random.default_rng(52)
    n, d, d_c, d_r = 3, 8, 3, 4
    h = rng.standard_normal((n, d))
    w_dkv = np.eye(d)[[5, 0, 2]]
    w_kr = np.eye(d)[[1, 3, 4, 7]]
    rows = mla.produce_rows(h, w_dkv, w_kr, None, 0.0, pos=np.zeros(n, dtype=int))
    np.testing.assert_array_equal(rows[:, :d_c], h[:, [5, 0, 2]])
    np.testing.assert_allclose(rows[:, d_c:], h[:, [1, 3, 4, 7]], rtol=0, atol=1e-15)
    pos = np.array([0, 7, 1000])
    rot = mla.produce_rows(h, w_dkv, w_kr, None, 0.0, pos=pos)
    np.testing.assert_allclose(rot[:, d_c:], rope(h[:, [1, 3, 4, 7]], pos), rtol=1e-13)
    # a rotation keeps the norm of each pair
    a = rot[:, d_c:].reshape(n, -1, 2)
    b = h[:, [1, 3, 4, 7]].reshape(n, -1, 2)
    np.testing.assert_allclose(np.linalg.norm(a, axis=2), np.linalg.norm(b, axis=2), rtol=1e-13)


# ------------------------------------------------- YaRN context extension
# DeepSeek-V2's settings ("DeepSeek-V2", section 3, long context extension):
# s = 40, alpha = 1, beta = 32 over a 4K training context, RoPE base 10^4,
# d_h^R = 64.
from oracle.rope import rope_theta, yarn_logit_factor, yarn_theta  # noqa: E402

V2_YARN = dict(base=10000.0, factor=40.0, alpha=1.0, beta=32.0, orig_len=4096)


def test_yarn_without_scaling_is_plain_rope():
    for s in (0.0, 0.5, 1.0):
        np.testing.assert_array_equal(yarn_theta(64, 10000.0, s, 1.0, 32.0, 4096),
                                      rope_theta(64))
    # and rope_theta is the frequency rope() uses by default
    x = np.random.default_rng(3).standard_normal((4, 64))
    p = np.array([0, 5, 999, 4095])
    np.testing.assert_array_equal(rope(x, p, theta=rope_theta(64)), rope(x, p))


def test_yarn_regimes_for_the_v2_settings():
    # Pair k turns r_k = 4096 * 10^(-k/8) / (2 pi) times over the 4K context.
    # r_k > beta = 32  <=>  k < 8 log10(4096 / (64 pi)) = 10.47: pairs 0..10 keep theta;
    # r_k < alpha = 1  <=>  k > 8 log10(4096 / (2 pi)) = 22.51: pairs 23..31 get theta / 40.
    th, t0 = yarn_theta(64, **V2_YARN), rope_theta(64)
    assert list(np.nonzero(th == t0)[0]) == list(range(0, 11))
    assert list(np.nonzero(np.abs(th * 40 / t0 - 1) < 1e-15)[0]) == list(range(23, 32))
    mid = np.arange(11, 23)
    assert np.all(th[mid] < t0[mid]) and np.all(th[mid] > t0[mid] / 40)


def test_yarn_ramp_is_monotone():
    ratio = yarn_theta(64, **V2_YARN) / rope_theta(64)
    assert np.all(np.diff(ratio) <= 1e-15)      # fewer turns -> closer to 1/s (up to rounding)
    assert ratio[0] == 1.0 and abs(ratio[-1] * 40 - 1) < 1e-15


def test_yarn_interpolates_low_and_keeps_high_frequencies():
    # Low-frequency pairs rotate at position s*p as plain RoPE does at p
    # (position interpolation); high-frequency pairs rotate exactly as
    # plain RoPE at the same position.
    th = yarn_theta(64, **V2_YARN)
    x = np.random.default_rng(4).standard_normal((5, 64))
    p = np.array([3, 77, 1000, 4095, 100])
    np.testing.assert_allclose(rope(x, 40 * p, theta=th)[:, 46:], rope(x, p)[:, 46:],
                               rtol=0, atol=1e-9)
    np.testing.assert_array_equal(rope(x, p, theta=th)[:, :22], rope(x, p)[:, :22])


def test_yarn_relative_position_property():
    th = yarn_theta(64, **V2_YARN)
    rng = np.random.default_rng(5)
    x, y = rng.standard_normal(64), rng.standard_normal(64)
    for m, n, k in ((100000, 99000, 98000), (160000, 5, 5), (7, 3, 2)):
        a = rope(x[None], np.array([m]), theta=th)[0] @ rope(y[None], np.array([n]), theta=th)[0]
        b = rope(x[None], np.array([m - k]), theta=th)[0] @ rope(y[None], np.array([n - k]), theta=th)[0]
        assert abs(a - b) <= 1e-9 * (abs(a) + 1)


def test_yarn_logit_factor_and_how_it_enters():
    assert yarn_logit_factor(1.0, 0.0707) == 1.0 and yarn_logit_factor(0.0, 0.1) == 1.0
    # sqrt(t) = 0.0707 ln 40 + 1 with ln 40 = 3.6888794541139363
    m = 0.0707 * 3.6888794541139363 + 1.0
    assert abs(yarn_logit_factor(40.0, 0.0707) - m * m) < 1e-14
    assert yarn_logit_factor(40.0, 0.1) > yarn_logit_factor(40.0, 0.0707) > 1.0
    # a factor t on the logits is the same as scaling the whole query by t
    rng = np.random.default_rng(6)
    H, dh, dc, dr, L = 2, 8, 16, 4, 9
    qn, qr = rng.standard_normal((1, H, dh)), rng.standard_normal((1, H, dr))
    wuk, wuv = rng.standard_normal((H, dh, dc)), rng.standard_normal((H, dh, dc))
    C, KR = rng.standard_normal((L, dc)), rng.standard_normal((L, dr))
    t = yarn_logit_factor(40.0, 0.0707)
    a = mla.decode(qn, qr, wuk, wuv, C, KR, [0], [L], 1, softmax_scale=t / math.sqrt(dh + dr))
    b = mla.decode(t * qn, t * qr, wuk, wuv, C, KR, [0], [L], 1)
    for k in ("o", "latent", "lse"):
        np.testing.assert_allclose(a[k], b[k], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------- 6-bit latent cache
def test_e2m3_values_are_the_e4m3_values_on_the_e2m3_grid():
    """E2M3 shares E4M3's 3 mantissa bits with a narrower exponent range: its
    non-negative values are exactly the E4M3 values v in [0, 7.5] with 8 v
    an integer (E2M3's subnormal spacing is 1/8).  The E4M3 side comes from
    torch's float8_e4m3fn, independent of the E2M3 table."""
    e4 = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    e4 = e4.numpy()
    grid = sorted(v for v in e4 if 0 <= v <= 7.5 and float(v * 8).is_integer())
    assert len(grid) == 32
    np.testing.assert_array_equal(formats.E2M3_TABLE[:32], np.array(grid))
    # sign bit: codes 32..63 are the negatives of 0..31
    np.testing.assert_array_equal(formats.E2M3_TABLE[32:], -formats.E2M3_TABLE[:32])


def test_e2m3_landmarks():
    t = formats.E2M3_TABLE
    assert t[0x1F] == 7.5 and t[0x01] == 0.125 and t[0x08] == 1.0 and t[0x3F] == -7.5
    assert t[0x07] == 0.875 and t[0x10] == 2.0 and t[0x18] == 4.0 and t[0x19] == 4.5


def test_mxfp6_golden_block():
    with open(os.path.join(GOLDEN, "mxfp6_block_example.json")) as f:
        g = json.load(f)
    row = np.zeros((1, 576), dtype=np.float32)
    row[0, :4] = g["block"]
    codes, exps = formats.quantize_rows_mxfp6(row)
    assert codes[0, :4].tolist() == g["expected_codes"]
    assert exps[0, 0] == g["expected_exponent"]
    assert np.all(exps[0, 1:] == g["expected_zero_block_exponent"])
    np.testing.assert_array_equal(formats.dequantize_rows_mxfp6(codes, exps)[0, :4],
                                  g["expected_values"])
    packed = formats.pack_rows_mxfp6(codes, exps)
    assert packed[0, :3].tolist() == g["expected_first_bytes"]
    assert packed[0, 432] == g["expected_exponent_byte"]
    assert packed.shape == (1, 452) and np.all(packed[0, 450:] == 0)


def test_mxfp6_quantisation_bounds_and_idempotence():
    """Per block: amax / 2^e lies in [4, 8); each element is within half a
    grid step of its stored value (the step of E2M3 at the element's
    magnitude, 1/8 below 2, 1/4 in [2, 4), 1/2 in [4, 8), times 2^e), or
    saturated at 7.5 * 2^e from below 8 * 2^e; quantising the stored values
    returns the same codes; codes are monotone in the input."""
    rng = np.random.default_rng(5)
    rows = (rng.standard_normal((64, 576)) * np.exp(rng.uniform(-6, 6, (64, 1)))).astype(np.float32)
    rows[3, :32] = 0.0                                   # an all-zero block
    codes, exps = formats.quantize_rows_mxfp6(rows)
    blocks = rows.astype(np.float64).reshape(64, 18, 32)
    amax = np.abs(blocks).max(axis=2)
    ratio = amax / np.ldexp(1.0, exps)
    nz = amax > 0
    assert np.all((ratio[nz] >= 4) & (ratio[nz] < 8))
    assert exps[3, 0] == -126
    deq = formats.dequantize_rows_mxfp6(codes, exps).reshape(64, 18, 32)
    y = np.abs(blocks) / np.ldexp(1.0, exps)[:, :, None]
    step = np.where(y < 2, 0.125, np.where(y < 4, 0.25, 0.5))
    err = np.abs(blocks - deq) / np.ldexp(1.0, exps)[:, :, None]
    sat = y > 7.5
    assert np.all(err[~sat] <= step[~sat] / 2 + 1e-12)
    assert np.all(err[sat] < 0.5)
    codes2, exps2 = formats.quantize_rows_mxfp6(deq.reshape(64, 576).astype(np.float32))
    np.testing.assert_array_equal(codes2, codes)
    xs = np.linspace(-7.5, 7.5, 4001)
    v = formats.e2m3_to_f64(formats.e2m3_nearest_sat(xs))
    assert np.all(np.diff(v) >= 0)


def test_mxfp6_packing_bit_order():
    """Code i of block k sits at bits 6 i .. 6 i + 5 of bytes 24 k .. 24 k + 23
    read as one little-endian integer; byte 432 + k is e_k + 127."""
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 64, (3, 576)).astype(np.uint8)
    exps = rng.integers(-126, 128, (3, 18)).astype(np.int32)
    packed = formats.pack_rows_mxfp6(codes, exps)
    for r in range(3):
        for k in range(18):
            word = int.from_bytes(bytes(packed[r, 24 * k:24 * k + 24]), "little")
            for i in range(32):
                assert (word >> (6 * i)) & 63 == codes[r, 32 * k + i]
            assert int(packed[r, 432 + k]) == exps[r, k] + 127


def test_mxfp6_bits_per_element():
    """The 6-bit cache: 576 codes of 6 bits plus 18 block exponents of 8 bits
    = 6.25 bits per element (the pages: about 6 bits per element on
    average); 452 bytes per token row with 2 bytes of padding."""
    assert (576 * 6 + 18 * 8) / 576 == 6.25
    assert formats.MXFP6_ROW_BYTES == 452 and 576 * 6 // 8 + 18 + 2 == 452
