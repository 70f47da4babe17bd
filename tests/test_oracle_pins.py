"""Pins of the CPU oracle to things other than itself: exact rational
arithmetic, closed forms, library routines (SVD, torch SDPA), hand-derived
fixtures and invariants. Each test names the oracle step it pins."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.qwm_oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f16_hex(h):
    return format(int(np.asarray(h, np.float16).view(np.uint16)), "04x")


def _fp16_grid():
    """All finite float16 values as Fractions, sorted."""
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    vals = vals[np.isfinite(vals)]
    vals = np.unique(vals.astype(np.float64))
    return vals


FP16_VALUES = _fp16_grid()


# ---------------------------------------------------------------- rounding helpers

def test_fp16_directed_rounding_exact():
    """fp16_round_down/up give the largest fp16 <= x / smallest fp16 >= x (exact search over all fp16)."""
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(3),
        (rng.standard_normal(500) * 1e-5).astype(np.float32),
        FP16_VALUES[(rng.integers(0, len(FP16_VALUES), 200))].astype(np.float32),
        np.array([0.0, -0.0, 65504.0, -65504.0, 6.1e-5, -6.1e-5], np.float32),
    ])
    dn = O.fp16_round_down(x).astype(np.float64)
    up = O.fp16_round_up(x).astype(np.float64)
    xd = x.astype(np.float64)
    i_dn = np.searchsorted(FP16_VALUES, xd, side="right") - 1
    i_up = np.searchsorted(FP16_VALUES, xd, side="left")
    assert np.array_equal(dn, FP16_VALUES[i_dn])
    assert np.array_equal(up, FP16_VALUES[i_up])


def test_fp16_step_up_exact():
    """fp16_step_up gives the smallest fp16 s >= x with 3 s an fp16 value
    (exhaustive search over the fp16 grid, exact float64 arithmetic):
    normal and subnormal steps, exact fp16 inputs (odd and even
    significands), values just above an fp16, and zero."""
    rng = np.random.default_rng(4)
    grid = FP16_VALUES[(FP16_VALUES >= 0) & (FP16_VALUES < 20000)]
    x = np.concatenate([
        np.abs(rng.standard_normal(3000)).astype(np.float32) * np.float32(2),
        (np.abs(rng.standard_normal(500)) * 1e-5).astype(np.float32),
        grid[rng.integers(0, len(grid), 1000)].astype(np.float32),
        np.nextafter(grid[rng.integers(0, len(grid), 300)].astype(np.float32), np.float32(np.inf)),
        np.array([0.0, 2.0 / 3.0, 1.0, 21824.0, 6.1e-5, 5.96e-8], np.float32),
    ])
    got = O.fp16_step_up(x).astype(np.float64)
    trip = set((3 * FP16_VALUES[FP16_VALUES >= 0]).tolist()) & set(FP16_VALUES.tolist())
    ok = np.array(sorted(v / 3 for v in trip))  # the fp16 steps whose triple is an fp16
    assert np.all(np.isin(ok, FP16_VALUES))
    want = ok[np.searchsorted(ok, x.astype(np.float64), side="left")]
    assert np.array_equal(got, want)
    # at most three ulps above plain upward rounding
    up = O.fp16_round_up(x)
    steps = (got.astype(np.float16).view(np.uint16).astype(np.int64) - up.view(np.uint16).astype(np.int64))
    assert steps.min() >= 0 and steps.max() <= 3


def test_f64_to_fp16_is_single_rounding():
    """float64 -> fp16 is one nearest-even rounding, including values just off a
    float16 midpoint that a float32 detour would round onto it."""
    rng = np.random.default_rng(2)
    base = FP16_VALUES[(FP16_VALUES > 1e-3) & (FP16_VALUES < 1e3)]
    a = base[rng.integers(0, len(base) - 1, 300)]
    idx = np.searchsorted(FP16_VALUES, a)
    b = FP16_VALUES[idx + 1]
    mid = (a + b) / 2
    cases = np.concatenate([mid, mid * (1 + 2.0 ** -40), mid * (1 - 2.0 ** -40),
                            rng.standard_normal(2000) * 10])
    got = O.f64_to_fp16(cases).astype(np.float64)
    for x, y in zip(cases, got):
        fx = Fraction(float(x))
        j = np.searchsorted(FP16_VALUES, x)
        lo = FP16_VALUES[max(j - 1, 0)]
        hi = FP16_VALUES[min(j, len(FP16_VALUES) - 1)]
        if Fraction(float(hi)) == fx:
            exp = hi
        else:
            dl = fx - Fraction(float(lo))
            dh = Fraction(float(hi)) - fx
            if dl < dh:
                exp = lo
            elif dh < dl:
                exp = hi
            else:
                lb = int(np.float16(lo).view(np.uint16))
                exp = lo if lb % 2 == 0 else hi
        assert y == exp, (x, y, exp)


def test_f64_to_bf16_is_single_rounding():
    """f64_to_bf16 equals exact nearest-even rounding to an 8-bit significand."""
    rng = np.random.default_rng(3)
    xs = list(rng.standard_normal(3000) * 5)
    # exact midpoints between adjacent bf16 values and values just off them
    for _ in range(300):
        v = np.float32(rng.standard_normal() * 4)
        u = int(v.view(np.uint32)) & 0xFFFF0000
        lo = float(np.uint32(u).view(np.float32))
        hi = float(np.uint32(u + 0x10000).view(np.float32))
        m = (lo + hi) / 2
        xs += [m, m + abs(m) * 2.0 ** -45, m - abs(m) * 2.0 ** -45]
    xs = np.array(xs, np.float64)
    got = O.f64_to_bf16(xs)
    for x, y in zip(xs, got):
        fx = Fraction(float(x))
        f32 = np.float32(x)
        u = int(f32.view(np.uint32)) & 0xFFFF0000
        cands = set()
        for du in (-0x10000, 0, 0x10000, 0x20000):
            uu = (u + du) & 0xFFFFFFFF
            c = np.uint32(uu).view(np.float32)
            if np.isfinite(c):
                cands.add(float(c))
        best = min(cands, key=lambda c: (abs(Fraction(c) - fx),
                                         (int(np.float32(c).view(np.uint32)) >> 16) & 1))
        assert float(y) == best, (x, y, best)


# ---------------------------------------------------------------- O1 sensitivity

def test_sensitivity_closed_form():
    """S_G = sum_{j in G} mean_i q_ij^2, hand-computed on a 2x4 example (g=2)."""
    q = np.array([[1, 2, 3, 4], [3, 4, 5, 6]], np.float32)
    # channel sums of squares: 10, 20, 34, 52 -> groups 30, 86 -> / M=2 -> 15, 43
    assert O.sensitivity(q, 2).tolist() == [15.0, 43.0]


def test_sensitivity_matches_rational_arithmetic():
    rng = np.random.default_rng(4)
    q = W.round_to_bf16(rng.standard_normal((37, 64)).astype(np.float32) * 3)
    S = O.sensitivity(q, 32)
    for G in range(2):
        tot = sum(Fraction(float(x)) ** 2 for x in q[:, G * 32:(G + 1) * 32].ravel())
        exact = tot / 37
        assert abs(Fraction(float(S[G])) - exact) <= exact * Fraction(1, 2 ** 24)


# ---------------------------------------------------------------- O2 QSAC objective

def _exact_J(k, c, S, g):
    tot = Fraction(0)
    for G in range(len(k) // g):
        r = [Fraction(float(a)) - Fraction(float(b)) for a, b in zip(k[G * g:(G + 1) * g], c[G * g:(G + 1) * g])]
        tot += Fraction(float(S[G])) * (max(r) - min(r)) ** 2
    return tot


def test_qsac_golden_fixture():
    """Hand-derived tiny case where QSAC and nearest-centroid disagree."""
    gd = _load("qsac_tiny.json")
    k = np.array(gd["k"], np.float32)
    C = np.array(gd["C"], np.float32)
    S = np.array(gd["S"], np.float32)
    g = gd["g"]
    assert O.qsac_objective(k, C, S, g).tolist() == gd["J"]
    assert O.qsac_assign(k, C, S, g).tolist() == gd["qsac_id"]
    assert O.nearest_assign(k, C).tolist() == gd["nearest_id"]
    for which, cid in (("forced_c0", 0), ("qsac", 1)):
        codes, zp, sc = O.int2_quantize(k - C[cid], g)
        assert codes.tolist() == gd[which]["codes"]
        assert [[_f16_hex(z) for z in row] for row in zp] == gd[which]["zp_f16_hex"]
        assert [[_f16_hex(s) for s in row] for row in sc] == gd[which]["scale_f16_hex"]


def test_qsac_brute_force_exact():
    """On tiny random inputs the float32 argmin equals the argmin of exactly
    computed J wherever the exact gap between the two best is not tiny, and
    the float32 J is within rounding of the exact J."""
    rng = np.random.default_rng(5)
    checked = 0
    for trial in range(12):
        d, g = 8, 4
        m = int(rng.integers(2, 9))
        N = 48
        k = rng.standard_normal((N, d)).astype(np.float32) * np.float32(2)
        C = rng.standard_normal((m, d)).astype(np.float32) * np.float32(2)
        S = (rng.random(d // g) * 3 + 0.1).astype(np.float32)
        J = O.qsac_objective(k, C, S, g)
        ids = O.qsac_assign(k, C, S, g)
        for n in range(N):
            ex = [_exact_J(k[n], C[c], S, g) for c in range(m)]
            for c in range(m):
                assert abs(Fraction(float(J[n, c])) - ex[c]) <= ex[c] * Fraction(1, 2 ** 20) + Fraction(1, 2 ** 60)
            order = sorted(range(m), key=lambda c: (ex[c], c))
            best, second = order[0], order[1]
            if ex[second] - ex[best] > ex[second] * Fraction(1, 10 ** 6):
                assert ids[n] == best
                checked += 1
    assert checked > 400


def test_qsac_tie_goes_to_smallest_id():
    rng = np.random.default_rng(6)
    k = rng.standard_normal((10, 64)).astype(np.float32)
    C = rng.standard_normal((6, 64)).astype(np.float32)
    C[4] = C[1]
    C[5] = C[1]
    S = np.ones(2, np.float32)
    J = O.qsac_objective(k, C, S, 32)
    ids = O.qsac_assign(k, C, S, 32)
    for n in range(10):
        assert J[n, ids[n]] == J[n].min()
        assert ids[n] == int(np.nonzero(J[n] == J[n].min())[0][0])
        assert ids[n] not in (4, 5)


def test_qsac_shift_invariance_and_group_weights():
    """J ignores a constant added to a centroid over one group (the zero-point
    absorbs it), and a zero-sensitivity group does not contribute."""
    rng = np.random.default_rng(7)
    k = (rng.integers(-64, 64, (20, 64)) / 8).astype(np.float32)
    C = (rng.integers(-64, 64, (5, 64)) / 8).astype(np.float32)
    S = np.array([2.0, 0.5], np.float32)
    J0 = O.qsac_objective(k, C, S, 32)
    C2 = C.copy()
    C2[:, 32:] += np.float32(1.25)  # dyadic shift: all arithmetic stays exact
    assert np.array_equal(O.qsac_objective(k, C2, S, 32), J0)
    # zero weight on group 1: J equals group-0 term alone
    S0 = np.array([2.0, 0.0], np.float32)
    Jg0 = O.qsac_objective(k, C, S0, 32)
    r = k[:, None, :32] - C[None, :, :32]
    rng_ = r.max(2) - r.min(2)
    assert np.array_equal(Jg0, np.float32(2.0) * rng_ * rng_)


def test_qsac_not_nearest_and_cuts_weighted_error():
    """On workload-shaped data QSAC differs from nearest-centroid assignment and
    lowers the sensitivity-weighted Key reconstruction error, the quantity the
    abstract says QSAC reduces ("quantization errors in channels that are more
    critical to attention")."""
    w = W.workload("tiny")
    hg = W.HeadGen(w, 0)
    keys = hg.cache_keys()
    qh = hg.hist_queries()
    S = O.sensitivity(qh, w.group)
    C = O.init_centroids(keys, w.n_centroids)
    s_ch = (qh.astype(np.float64) ** 2).mean(0)

    def weighted_err(ids):
        r = keys - C[ids]
        codes, zp, sc = O.int2_quantize(r, w.group)
        rh = O.int2_dequant64(codes, zp, sc, w.group)
        return float((((r.astype(np.float64) - rh) ** 2) * s_ch).sum(1).mean())

    ids_q = O.qsac_assign(keys, C, S, w.group)
    ids_n = O.nearest_assign(keys, C)
    assert np.mean(ids_q != ids_n) > 0.05
    assert weighted_err(ids_q) < 0.97 * weighted_err(ids_n)


# ---------------------------------------------------------------- O4/O5 INT2

def test_int2_half_step_bound_and_coverage():
    """The stored grid covers [mn, mx] (exact comparison), zp is the largest
    fp16 <= mn, scale the smallest fp16 >= (mx - zp)/3 whose triple is an
    fp16, and every element is within half a step (plus float32 rounding) of
    its reconstruction."""
    rng = np.random.default_rng(8)
    x = np.concatenate([
        rng.standard_normal((300, 128)).astype(np.float32) * np.float32(4),
        (rng.standard_normal((50, 128)) * 1e-4).astype(np.float32),
        (rng.standard_normal((50, 128)) * 50).astype(np.float32),
    ])
    codes, zp, sc = O.int2_quantize(x, 32)
    rh = O.int2_dequant(codes, zp, sc, 32)
    xg = x.reshape(len(x), 4, 32).astype(np.float64)
    zpf = zp.astype(np.float64)
    scf = sc.astype(np.float64)
    assert np.all(zpf <= xg.min(2))
    # the top of the grid reaches mx up to the float32 rounding of the step
    # computation (mx - zp) / 3: two float32 ulps of mx - zp
    span = xg.max(2) - zpf
    assert np.all(zpf + 3 * scf >= xg.max(2) - 2 * span * 2.0 ** -24)
    nxt = np.nextafter(zp, np.float16(np.inf)).astype(np.float64)
    assert np.all(nxt > xg.min(2))
    step32 = ((xg.max(2).astype(np.float32) - zp.astype(np.float32)) / np.float32(3)).astype(np.float64)
    assert np.all(scf >= step32)
    # minimal among the fp16 values >= step32 whose triple is an fp16
    assert np.all(np.isin(3 * scf, FP16_VALUES))
    for want, got in zip(step32.ravel(), scf.ravel()):
        i = np.searchsorted(FP16_VALUES, want, side="left")
        while not np.isin(3 * FP16_VALUES[i], FP16_VALUES):
            i += 1
        assert got == FP16_VALUES[i]
    err = np.abs(x.astype(np.float64) - rh.astype(np.float64)).reshape(len(x), 4, 32)
    mag = np.maximum(np.abs(xg), np.abs(zpf)[:, :, None] + 3 * scf[:, :, None])
    bound = scf[:, :, None] / 2 + 4 * mag * 2.0 ** -24
    assert np.all(err <= bound)
    assert codes.max() <= 3


def test_int2_half_integer_ties_golden():
    """Hand-derived fixture (tests/golden/int2_ties.json): quotients of exactly
    0.5, 1.5 and 2.5 go to the even code (0, 2, 2). Run through the plain
    quantizer and through quantize-on-insert, as the Key residual (one
    all-zero centroid, so r = k) and as the Value."""
    fx = _load("int2_ties.json")
    x = np.array(fx["x"], np.float32)
    codes, zp, sc = O.int2_quantize(x, fx["g"])
    assert codes.tolist() == fx["codes"]
    assert [[_f16_hex(v) for v in row] for row in zp] == fx["zp_f16_hex"]
    assert [[_f16_hex(v) for v in row] for row in sc] == fx["step_f16_hex"]
    d = x.shape[1]
    rec = O.quantize_tokens(x, x, np.zeros((1, d), np.float32), np.ones(d // fx["g"], np.float32),
                            np.zeros((d, 0), np.float32), fx["g"])
    for code_f, zp_f, sc_f in (("kcode", "kzp", "kscale"), ("vcode", "vzp", "vscale")):
        assert rec[code_f].tolist() == fx["codes"]
        assert [[_f16_hex(v) for v in row] for row in rec[zp_f]] == fx["zp_f16_hex"]
        assert [[_f16_hex(v) for v in row] for row in rec[sc_f]] == fx["step_f16_hex"]


def test_int2_grid_values_reproduce_exactly():
    """Values built on a fp16-exact grid with codes 0 and 3 present in every
    group come back bit for bit; constant groups give scale 0 and codes 0."""
    rng = np.random.default_rng(9)
    N, d, g = 64, 128, 32
    zp = (rng.integers(-512, 512, (N, d // g)) / 64).astype(np.float16)
    sc = (rng.integers(1, 256, (N, d // g)) / 128).astype(np.float16)
    codes = rng.integers(0, 4, (N, d)).astype(np.uint8)
    cg = codes.reshape(N, d // g, g)
    cg[:, :, 0] = 0
    cg[:, :, 1] = 3
    x = O.int2_dequant(codes, zp, sc, g)
    c2, z2, s2 = O.int2_quantize(x, g)
    assert np.array_equal(c2, codes)
    assert np.array_equal(z2.view(np.uint16), zp.view(np.uint16))
    assert np.array_equal(s2.view(np.uint16), sc.view(np.uint16))
    const = np.repeat(np.float32([0.75, -2.5, 0.0, 3.0]), 32)[None, :].repeat(3, 0)
    c3, z3, s3 = O.int2_quantize(const, g)
    assert np.all(c3 == 0) and np.all(s3.view(np.uint16) == 0)
    assert np.array_equal(O.int2_dequant(c3, z3, s3, g), const)


def test_int2_signed_zero_canonical():
    x = np.zeros((2, 32), np.float32)
    x[1] = -0.0
    _, zp, sc = O.int2_quantize(x, 32)
    assert np.all(zp.view(np.uint16) == 0) and np.all(sc.view(np.uint16) == 0)


def test_pack_golden_and_roundtrip():
    gd = _load("pack_tiny.json")
    codes = np.array(gd["codes"], np.uint8)
    assert O.pack2(codes).tolist() == gd["packed"]
    rng = np.random.default_rng(10)
    c = rng.integers(0, 4, (33, 128)).astype(np.uint8)
    assert np.array_equal(O.unpack2(O.pack2(c)), c)


# ---------------------------------------------------------------- O6 PSAC basis

def test_subspace_projector_matches_svd():
    """U_r from the Gram eigendecomposition spans the same subspace as the
    top-r right singular vectors of Q (numpy SVD), and the sign rule holds."""
    w = W.workload("video_chunk")
    hg = W.HeadGen(w, 3)
    q = hg.hist_queries()
    U = O.subspace(q, 8).astype(np.float64)
    _, _, vt = np.linalg.svd(q.astype(np.float64), full_matrices=False)
    P1 = U @ U.T
    P2 = vt[:8].T @ vt[:8]
    assert np.linalg.norm(P1 - P2) / np.linalg.norm(P2) < 1e-5
    assert np.allclose(U.T @ U, np.eye(8), atol=1e-6)
    for k in range(8):
        i = int(np.argmax(np.abs(U[:, k])))
        assert U[i, k] > 0


def test_query_energy_matches_article():
    """The synthetic Queries put about 70% of their energy in the first 8
    principal directions (article, 'Step 2': about 71% for one layer)."""
    w = W.workload("wm_layer")
    q = W.HeadGen(w, 0).hist_queries().astype(np.float64)
    ev = np.linalg.eigvalsh(q.T @ q)[::-1]
    frac = ev[:8].sum() / ev.sum()
    assert 0.66 < frac < 0.74


# ---------------------------------------------------------------- O7/O9 PSAC + attention

def _head_cache(k, v, q_hist, m, r, g, dtype="f32", iters=3):
    S = O.sensitivity(q_hist, g)
    U = O.subspace(q_hist, r)
    C = O.build_centroids(k, S, m, g, iters, dtype)
    hc = O.HeadCache(g, dtype)
    hc.add_epoch(C, S, U)
    hc.append(k, v)
    return hc, (C, S, U)


def test_psac_full_rank_restores_exact_logits():
    """With r = d the compensated logits equal q.k up to the fp16 rounding of
    the coefficients (bound: sum |qU| * half-ulp(coef))."""
    rng = np.random.default_rng(11)
    d = 64
    k = rng.standard_normal((200, d)).astype(np.float32) * np.float32(2)
    v = rng.standard_normal((200, d)).astype(np.float32)
    qh = rng.standard_normal((300, d)).astype(np.float32)
    hc, (C, S, U) = _head_cache(k, v, qh, 8, d, 32)
    q = rng.standard_normal((7, d)).astype(np.float64)
    got = O.cache_logits(q, hc, 1.0)
    exact = q @ k.astype(np.float64).T
    coef = hc.field("coef").astype(np.float64)
    half_ulp = np.maximum(np.abs(coef) * 2.0 ** -11, 2.0 ** -25)
    qu = np.abs(q @ U.astype(np.float64))
    bound = qu @ half_ulp.T + 1e-9 * np.abs(exact).max()
    assert np.all(np.abs(got - exact) <= bound)
    # and far below the error without compensation
    nocomp = q @ hc.khat64().T
    assert np.abs(got - exact).max() < 0.05 * np.abs(nocomp - exact).max()


def test_psac_exact_for_queries_in_subspace():
    """Queries inside span(U_r) see exact logits at any rank r, because
    q U U^T e = q e for such q."""
    rng = np.random.default_rng(12)
    d, r = 64, 4
    k = rng.standard_normal((150, d)).astype(np.float32) * np.float32(2)
    v = rng.standard_normal((150, d)).astype(np.float32)
    qh = rng.standard_normal((100, d)).astype(np.float32)
    hc, (C, S, U) = _head_cache(k, v, qh, 4, r, 32)
    Uq = np.linalg.qr(U.astype(np.float64))[0]
    q = rng.standard_normal((5, r)) @ Uq.T
    got = O.cache_logits(q, hc, 1.0)
    exact = q @ k.astype(np.float64).T
    coef = hc.field("coef").astype(np.float64)
    qu = np.abs(q @ U.astype(np.float64))
    e_off = np.abs(q @ (np.eye(d) - U.astype(np.float64) @ U.astype(np.float64).T)).sum(1, keepdims=True)
    bound = qu @ np.maximum(np.abs(coef) * 2.0 ** -11, 2.0 ** -25).T + e_off * 1e-3 + 1e-9
    assert np.all(np.abs(got - exact) <= bound)


def _grid_cache(rng, N, d, g, m, r):
    """A cache whose Keys/Values sit exactly on their quantization grid, so the
    quantization error is zero (keys = c_id + zp + code*scale)."""
    C = (rng.integers(-40, 40, (m, d)) * 8).astype(np.float32)  # far apart centroids
    ids = rng.integers(0, m, N)
    zp = (rng.integers(-64, 64, (N, d // g)) / 32).astype(np.float16)
    sc = (rng.integers(1, 32, (N, d // g)) / 64).astype(np.float16)
    codes = rng.integers(0, 4, (N, d)).astype(np.uint8)
    cg = codes.reshape(N, d // g, g)
    cg[:, :, 0] = 0
    cg[:, :, 1] = 3
    k = C[ids] + O.int2_dequant(codes, zp, sc, g)
    vz = (rng.integers(-64, 64, (N, d // g)) / 32).astype(np.float16)
    vs = (rng.integers(1, 32, (N, d // g)) / 64).astype(np.float16)
    vcodes = rng.integers(0, 4, (N, d)).astype(np.uint8)
    vg = vcodes.reshape(N, d // g, g)
    vg[:, :, 0] = 0
    vg[:, :, 1] = 3
    v = O.int2_dequant(vcodes, vz, vs, g)
    return C, ids, k, v


def test_grid_keys_reproduce_and_attention_is_textbook():
    """Keys built on the grid around their centroid come back with the same
    centroid id and zero error; attention then equals float64
    softmax(QK^T/sqrt(d))V from torch's SDPA, with and without a causal self
    segment."""
    rng = np.random.default_rng(13)
    N, d, g, m, r = 96, 64, 32, 6, 4
    C, ids, k, v = _grid_cache(rng, N, d, g, m, r)
    qh = rng.standard_normal((50, d)).astype(np.float32)
    S = O.sensitivity(qh, g)
    U = O.subspace(qh, r)
    hc = O.HeadCache(g, "f32")
    hc.add_epoch(C, S, U)
    hc.append(k, v)
    assert np.array_equal(hc.field("ids"), ids.astype(np.uint8))
    assert np.all(hc.field("coef").view(np.uint16) & 0x7FFF == 0)
    assert np.array_equal(hc.khat64(), k.astype(np.float64))
    q = rng.standard_normal((9, d))
    out = O.attend(q, hc)
    tq = torch.from_numpy(q)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, torch.from_numpy(k.astype(np.float64))[None, None],
        torch.from_numpy(v.astype(np.float64))[None, None])[0, 0].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    # causal self segment of 9 tokens appended after the cache
    ks = rng.standard_normal((9, d))
    vs = rng.standard_normal((9, d))
    out2 = O.attend(q, hc, ks, vs, mask="causal")
    kk = np.concatenate([k.astype(np.float64), ks])
    vv = np.concatenate([v.astype(np.float64), vs])
    allowed = np.ones((9, N + 9), bool)
    allowed[:, N:] = np.tril(np.ones((9, 9), bool))
    ref2 = torch.nn.functional.scaled_dot_product_attention(
        tq, torch.from_numpy(kk)[None, None], torch.from_numpy(vv)[None, None],
        attn_mask=torch.from_numpy(allowed)[None, None])[0, 0].numpy()
    assert np.allclose(out2, ref2, rtol=1e-12, atol=1e-12)


def test_attention_invariants():
    """Permuting cache tokens leaves the output unchanged; two halves merged by
    log-sum-exp equal the whole; softmax rows sum to one."""
    w = W.workload("tiny")
    hg = W.HeadGen(w, 0)
    k, v = hg.cache_keys(), hg.cache_values()
    qh = hg.hist_queries()
    q = hg.current_queries().astype(np.float64)
    S = O.sensitivity(qh, w.group)
    U = O.subspace(qh, w.rank)
    C = O.build_centroids(k, S, w.n_centroids, w.group, 2, "f32")
    full = O.HeadCache(w.group, "f32")
    full.add_epoch(C, S, U)
    full.append(k, v)
    out = O.attend(q, full)
    perm = np.random.default_rng(14).permutation(len(k))
    pc = O.HeadCache(w.group, "f32")
    pc.add_epoch(C, S, U)
    pc.append(k[perm], v[perm])
    assert np.allclose(O.attend(q, pc), out, rtol=1e-12, atol=1e-13)
    # LSE merge of halves
    parts = []
    for sl in (slice(0, 400), slice(400, None)):
        hc = O.HeadCache(w.group, "f32")
        hc.add_epoch(C, S, U)
        hc.append(k[sl], v[sl])
        ell = O.cache_logits(q, hc, 1 / np.sqrt(w.head_dim))
        mx = ell.max(1, keepdims=True)
        pe = np.exp(ell - mx)
        parts.append((mx, pe.sum(1, keepdims=True), pe @ hc.vhat64()))
    M = np.maximum(parts[0][0], parts[1][0])
    L = sum(l * np.exp(mx - M) for mx, l, _ in parts)
    Ov = sum(o * np.exp(mx - M) for mx, _, o in parts)
    assert np.allclose(Ov / L, out, rtol=1e-12, atol=1e-13)
    ell = O.cache_logits(q, full, 1 / np.sqrt(w.head_dim))
    p = np.exp(ell - ell.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    assert np.allclose(p.sum(1), 1.0)


def test_append_in_one_call_equals_per_frame():
    rng = np.random.default_rng(15)
    k = rng.standard_normal((300, 64)).astype(np.float32)
    v = rng.standard_normal((300, 64)).astype(np.float32)
    qh = rng.standard_normal((40, 64)).astype(np.float32)
    S, U = O.sensitivity(qh, 32), O.subspace(qh, 4)
    C = O.init_centroids(k, 8)
    a = O.HeadCache(32, "f32")
    a.add_epoch(C, S, U)
    a.append(k, v)
    b = O.HeadCache(32, "f32")
    b.add_epoch(C, S, U)
    for s in range(0, 300, 70):
        b.append(k[s:s + 70], v[s:s + 70])
    for f in ("ids", "kcode", "kzp", "kscale", "vcode", "vzp", "vscale", "coef"):
        assert np.array_equal(a.field(f).view(np.uint8), b.field(f).view(np.uint8)), f


def test_compensation_and_qsac_cut_top1_selection_change():
    """The article's Table 1 measures how often a Query's top-scoring cached
    token changes relative to full precision. On workload-shaped data,
    QSAC+PSAC changes fewer top-1 selections than nearest-centroid
    assignment without compensation."""
    w = W.workload("tiny")
    hg = W.HeadGen(w, 0)
    k, v = hg.cache_keys(), hg.cache_values()
    qh = hg.hist_queries()
    q = hg.queries(5, 256).astype(np.float64)
    S, U = O.sensitivity(qh, w.group), O.subspace(qh, w.rank)
    C = O.build_centroids(k, S, w.n_centroids, w.group, 5, "f32")
    hc = O.HeadCache(w.group, "f32")
    hc.add_epoch(C, S, U)
    hc.append(k, v)
    top_ref = np.argmax(q @ k.astype(np.float64).T, 1)
    top_qw = np.argmax(O.cache_logits(q, hc, 1.0), 1)
    # nearest-centroid residual quantization, no compensation
    ids = O.nearest_assign(k, C)
    codes, zp, sc = O.int2_quantize(k - C[ids], w.group)
    kh = C[ids].astype(np.float64) + O.int2_dequant64(codes, zp, sc, w.group)
    top_nn = np.argmax(q @ kh.T, 1)
    assert np.mean(top_qw != top_ref) < np.mean(top_nn != top_ref)


# ---------------------------------------------------------------- O3 centroids

def test_centroid_build_rules():
    """Init takes Key floor(i*N/m); the update is the mean rounded to the stored
    dtype; an empty cluster keeps its centroid."""
    k = np.array([[0, 0], [0, 2], [10, 10], [10, 12], [50, 50]], np.float32).repeat(16, 1)
    k = k.reshape(5, 32)
    S = np.ones(1, np.float32)
    C0 = O.init_centroids(k, 3)
    assert np.array_equal(C0, k[[0, 1, 3]])
    # with one iteration: assignment by QSAC; all rows are constant over the
    # group pattern [a,b,a,b...] so ranges decide
    C1 = O.build_centroids(k, S, 3, 32, 1, "f32")
    ids = O.qsac_assign(k, C0, S, 32)
    for i in range(3):
        sel = k[ids == i]
        if len(sel):
            assert np.array_equal(C1[i], sel.astype(np.float64).mean(0).astype(np.float32))
        else:
            assert np.array_equal(C1[i], C0[i])
    # empty cluster: duplicate seed never wins (ties go to the smaller id)
    kk = np.array([[1.0] * 32, [1.0] * 32, [5.0] * 32], np.float32)
    kk[2, 0] = 9.0
    Cb = O.build_centroids(kk, S, 3, 32, 1, "f32")
    assert np.array_equal(Cb[1], kk[1])  # seed of cluster 1 = key 1, tied with cluster 0 -> empty


def test_centroid_build_recovers_separated_means():
    rng = np.random.default_rng(16)
    d, comps = 64, 4
    mu = rng.standard_normal((comps, d)).astype(np.float32) * np.float32(30)
    lab = np.repeat(np.arange(comps), 200)
    rng.shuffle(lab)
    k = (mu[lab] + rng.standard_normal((len(lab), d)).astype(np.float32) * np.float32(0.1)).astype(np.float32)
    S = np.ones(2, np.float32)
    C = O.build_centroids(k, S, comps, 32, 10, "f32")
    ids = O.qsac_assign(k, C, S, 32)
    # each recovered cluster is one generating component
    for i in range(comps):
        assert len(set(lab[ids == i])) == 1
    # centroid equals the component's empirical mean up to rounding
    for i in range(comps):
        emp = k[ids == i].astype(np.float64).mean(0)
        assert np.allclose(C[i], emp, atol=1e-5)


def test_bf16_centroids_are_bf16():
    w = W.workload("video_chunk")
    hg = W.HeadGen(w, 1)
    k = hg.keys(0, 880)
    S = O.sensitivity(hg.hist_queries(), w.group)
    C = O.build_centroids(k, S, 16, w.group, 2, "bf16")
    assert np.all(C.view(np.uint32) & 0xFFFF == 0)


# ---------------------------------------------------------------- accounting

def test_compression_accounting_hand_values():
    """Bytes per token-head and the compression ratio, hand-computed.
    d=64, r=4: 2*16 codes + 2*2*4 params + 1 id + 2*4 coef = 57 B.
    tiny: 1024 tokens * 256 B bf16 / (1024*57 + 16*64*4 + 2*4 + 64*4*4) = 262144/63496.
    d=128, r=8: 64 + 32 + 1 + 16 = 113 B; video_chunk:
    7040*512 / (7040*113 + 64*128*2 + 16 + 128*8*4) = 3604480/816016."""
    assert O.bytes_per_token_head(64, 32, 4) == 57
    assert O.bytes_per_token_head(128, 32, 8) == 113
    assert O.bytes_per_token_head(128, 32, 16) == 129
    assert O.compression_ratio(1024, 64, 32, 16, 4, 4) == pytest.approx(262144 / 63496)
    assert O.compression_ratio(7040, 128, 32, 64, 8, 2) == pytest.approx(3604480 / 816016)
