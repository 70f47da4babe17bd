"""Pins of the oracle's baseline modes and of the top-1 diagnostic: QVG's
nearest-centroid rule (the baseline the article's "Step 1" compares QSAC
with), PSAC switched off (rank 0), and the share of Queries whose
top-scoring historical token changes against full precision (the article's
"Table 1"). Each test names the oracle function it pins and what it is pinned
to: exact rational arithmetic, a hand-derived fixture, closed forms or
textbook attention."""

import json
import os
from fractions import Fraction

import numpy as np
import torch

import oracle.qwm_oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _exact_D(k, c):
    return sum((Fraction(float(a)) - Fraction(float(b))) ** 2 for a, b in zip(k, c))


# ---------------------------------------------------------------- nearest centroid (QVG)

def test_nearest_golden_fixture():
    """The hand-derived fixture where QSAC and the nearest centroid disagree:
    squared distances 2 and 9, nearest id 0 (QSAC picks 1)."""
    with open(os.path.join(GOLDEN, "qsac_tiny.json")) as f:
        gd = json.load(f)
    k = np.array(gd["k"], np.float32)
    C = np.array(gd["C"], np.float32)
    assert O.nearest_objective(k, C, gd["g"]).tolist() == gd["nearest_D"]
    assert O.nearest_assign32(k, C, gd["g"]).tolist() == gd["nearest_id"]
    assert O.assign(k, C, np.array(gd["S"], np.float32), gd["g"], "qsac").tolist() == gd["qsac_id"]


def test_nearest_brute_force_exact():
    """nearest_objective is the squared distance within float32 rounding of the
    exact rational value, and its argmin is the exact argmin wherever the two
    best are not within 1e-6 relative of each other."""
    rng = np.random.default_rng(21)
    checked = 0
    for trial in range(10):
        d, g = 8, 4
        m = int(rng.integers(2, 9))
        N = 40
        k = rng.standard_normal((N, d)).astype(np.float32) * np.float32(3)
        C = rng.standard_normal((m, d)).astype(np.float32) * np.float32(3)
        D = O.nearest_objective(k, C, g)
        ids = O.nearest_assign32(k, C, g)
        for n in range(N):
            ex = [_exact_D(k[n], C[c]) for c in range(m)]
            for c in range(m):
                # d terms, each rounded twice (difference, square) plus the sums
                assert abs(Fraction(float(D[n, c])) - ex[c]) <= ex[c] * Fraction(3 * d, 2 ** 24) + Fraction(1, 2 ** 60)
            order = sorted(range(m), key=lambda c: (ex[c], c))
            if ex[order[1]] - ex[order[0]] > ex[order[1]] * Fraction(1, 10 ** 6):
                assert ids[n] == order[0]
                checked += 1
    assert checked > 300


def test_nearest_exact_on_dyadic_data_and_ties():
    """With small dyadic values every float32 operation is exact, so the cost
    equals the integer squared distance computed by hand, and equal distances
    go to the smallest id."""
    k = np.array([[1, 2, 0, -1, 3, 0, 0, 2]], np.float32) / np.float32(4)
    C = np.array([[0, 0, 0, 0, 0, 0, 0, 0],       # 1+4+0+1+9+0+0+4 = 19 -> 19/16
                  [1, 2, 0, -1, 3, 0, 0, 0],      # 4 -> 4/16
                  [1, 2, 0, -1, 3, 0, 0, 4],      # 4 -> 4/16 (tie with id 1)
                  [1, 2, 0, -1, 3, 0, 0, 2]],     # 0
                 np.float32) / np.float32(4)
    D = O.nearest_objective(k, C, 4)
    assert D.tolist() == [[19 / 16, 4 / 16, 4 / 16, 0.0]]
    assert O.nearest_assign32(k, C[:3], 4).tolist() == [1]
    assert O.nearest_assign32(k, C, 4).tolist() == [3]


def test_nearest_differs_from_qsac_and_qsac_wins_its_objective():
    """On workload-shaped data the two rules disagree on many Keys; each rule's
    choice is optimal for its own cost (QSAC's J is never above J of the
    nearest centroid, and vice versa for the distance)."""
    w = W.workload("tiny")
    hg = W.HeadGen(w, 0)
    keys = hg.cache_keys()
    S = O.sensitivity(hg.hist_queries(), w.group)
    C = O.init_centroids(keys, w.n_centroids)
    iq = O.assign(keys, C, S, w.group, "qsac")
    inn = O.assign(keys, C, S, w.group, "nearest")
    assert np.mean(iq != inn) > 0.05
    J = O.qsac_objective(keys, C, S, w.group)
    D = O.nearest_objective(keys, C, w.group)
    n = np.arange(len(keys))
    assert np.all(J[n, iq] <= J[n, inn])
    assert np.all(D[n, inn] <= D[n, iq])
    # the float32 rule agrees with the float64 nearest centroid away from near-ties
    D64 = ((keys[:, None, :].astype(np.float64) - C[None].astype(np.float64)) ** 2).sum(2)
    s = np.sort(D64, 1)
    clear = (s[:, 1] - s[:, 0]) > 1e-5 * s[:, 1]
    assert np.array_equal(inn[clear], O.nearest_assign(keys, C)[clear])


def test_nearest_build_recovers_separated_means():
    """Lloyd's algorithm with the nearest-centroid rule recovers well separated
    components and their empirical means (the textbook k-means fixed point)."""
    rng = np.random.default_rng(22)
    d, comps = 64, 4
    mu = rng.standard_normal((comps, d)).astype(np.float32) * np.float32(30)
    lab = np.repeat(np.arange(comps), 150)
    rng.shuffle(lab)
    k = (mu[lab] + rng.standard_normal((len(lab), d)).astype(np.float32) * np.float32(0.1)).astype(np.float32)
    S = np.zeros(2, np.float32)
    C = O.build_centroids(k, S, comps, 32, 10, "f32", objective="nearest")
    ids = O.nearest_assign32(k, C, 32)
    for i in range(comps):
        assert len(set(lab[ids == i])) == 1
        assert np.allclose(C[i], k[ids == i].astype(np.float64).mean(0), atol=1e-5)


# ---------------------------------------------------------------- PSAC off (rank 0)

def test_rank_zero_stores_no_coefficients_and_keeps_codes():
    """Rank 0 changes nothing but the coefficients: ids, codes and parameters
    equal those at rank 4, and no coefficient is stored."""
    w = W.workload("tiny")
    hg = W.HeadGen(w, 0)
    k, v = hg.cache_keys()[:300], hg.cache_values()[:300]
    qh = hg.hist_queries()
    S = O.sensitivity(qh, w.group)
    C = O.init_centroids(k, w.n_centroids)
    U4 = O.subspace(qh, 4)
    U0 = O.subspace(qh, 0)
    assert U0.shape == (w.head_dim, 0)
    for obj in O.OBJECTIVES:
        a = O.quantize_tokens(k, v, C, S, U4, w.group, obj)
        b = O.quantize_tokens(k, v, C, S, U0, w.group, obj)
        assert b["coef"].shape == (300, 0)
        for f in ("ids", "kcode", "kzp", "kscale", "vcode", "vzp", "vscale"):
            assert np.array_equal(a[f].view(np.uint8), b[f].view(np.uint8)), (obj, f)
    assert O.bytes_per_token_head(128, 32, 0) == 2 * 32 + 8 * 4 + 1
    assert O.bytes_per_token_head(64, 32, 0) == 2 * 16 + 8 * 2 + 1


def test_rank_zero_attention_is_textbook_on_grid_keys():
    """With zero quantization error, attention without compensation equals
    float64 softmax(QK^T/sqrt(d))V from torch's SDPA, for both rules."""
    rng = np.random.default_rng(23)
    N, d, g, m = 80, 64, 32, 5
    C = (rng.integers(-40, 40, (m, d)) * 8).astype(np.float32)
    ids = rng.integers(0, m, N)
    zp = (rng.integers(-64, 64, (N, d // g)) / 32).astype(np.float16)
    sc = (rng.integers(1, 32, (N, d // g)) / 64).astype(np.float16)
    codes = rng.integers(0, 4, (N, d)).astype(np.uint8)
    codes.reshape(N, d // g, g)[:, :, 0] = 0
    codes.reshape(N, d // g, g)[:, :, 1] = 3
    k = C[ids] + O.int2_dequant(codes, zp, sc, g)
    v = rng.standard_normal((N, d)).astype(np.float32)
    qh = rng.standard_normal((40, d)).astype(np.float32)
    for obj in O.OBJECTIVES:
        hc = O.HeadCache(g, "f32", obj)
        hc.add_epoch(C, O.sensitivity(qh, g), O.subspace(qh, 0))
        hc.append(k, v)
        assert np.array_equal(hc.field("ids"), ids.astype(np.uint8))
        assert np.array_equal(hc.khat64(), k.astype(np.float64))
        q = rng.standard_normal((7, d))
        # Values are INT2: compare against SDPA over the stored Values
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None], torch.from_numpy(k.astype(np.float64))[None, None],
            torch.from_numpy(hc.vhat64())[None, None])[0, 0].numpy()
        assert np.allclose(O.attend(q, hc), ref, rtol=1e-12, atol=1e-12)


def test_rank_zero_logits_are_uncompensated():
    """At rank 0 the logits are q . khat exactly; compensation at rank d brings
    them to q . k (so the rank-0 error is the full quantization error)."""
    rng = np.random.default_rng(24)
    d = 64
    k = rng.standard_normal((120, d)).astype(np.float32) * np.float32(2)
    v = rng.standard_normal((120, d)).astype(np.float32)
    qh = rng.standard_normal((200, d)).astype(np.float32)
    S = O.sensitivity(qh, 32)
    C = O.build_centroids(k, S, 6, 32, 2, "f32")
    h0 = O.HeadCache(32, "f32")
    h0.add_epoch(C, S, O.subspace(qh, 0))
    h0.append(k, v)
    hd = O.HeadCache(32, "f32")
    hd.add_epoch(C, S, O.subspace(qh, d))
    hd.append(k, v)
    q = rng.standard_normal((6, d))
    l0 = O.cache_logits(q, h0, 1.0)
    # with no coefficients the compensation term is empty
    assert np.array_equal(l0, q @ h0.khat64().T)
    exact = q @ k.astype(np.float64).T
    assert np.abs(O.cache_logits(q, hd, 1.0) - exact).max() < 0.05 * np.abs(l0 - exact).max()


# ---------------------------------------------------------------- top-1 diagnostic

def test_top1_brute_force_with_ties():
    """Integer Queries and Keys make every dot product exact: the top-1 index
    equals a hand loop's first maximum, ties included."""
    rng = np.random.default_rng(25)
    q = rng.integers(-3, 4, (30, 8)).astype(np.float64)
    k = rng.integers(-2, 3, (25, 8)).astype(np.float32)
    k[7] = k[3]  # exact ties: the earlier token must win
    k[20] = k[11]
    got = O.top1_dense(q, k)
    for i in range(30):
        best, bi = None, -1
        for j in range(25):
            s = sum(int(q[i, c]) * int(k[j, c]) for c in range(8))
            if best is None or s > best:
                best, bi = s, j
        assert got[i] == bi


def test_top1_cached_matches_dense_without_error_and_flags_a_change():
    """With zero quantization error the cached top-1 equals the full-precision
    top-1 (change rate 0). Moving one Key off its grid so that it overtakes the
    winner of one Query changes exactly that Query's top-1."""
    rng = np.random.default_rng(26)
    N, d, g, m = 60, 64, 32, 4
    C = (rng.integers(-8, 8, (m, d)) * 2).astype(np.float32)
    ids = rng.integers(0, m, N)
    zp = (rng.integers(-16, 16, (N, d // g)) / 8).astype(np.float16)
    sc = (rng.integers(1, 8, (N, d // g)) / 8).astype(np.float16)
    codes = rng.integers(0, 4, (N, d)).astype(np.uint8)
    codes.reshape(N, d // g, g)[:, :, 0] = 0
    codes.reshape(N, d // g, g)[:, :, 1] = 3
    k = C[ids] + O.int2_dequant(codes, zp, sc, g)
    v = rng.standard_normal((N, d)).astype(np.float32)
    qh = rng.standard_normal((30, d)).astype(np.float32)
    hc = O.HeadCache(g, "f32")
    hc.add_epoch(C, O.sensitivity(qh, g), O.subspace(qh, 0))
    hc.append(k, v)
    q = rng.integers(-2, 3, (12, d)).astype(np.float64)
    assert O.top1_change_rate(q, k, hc) == 0.0
    assert np.array_equal(O.top1_cached(q, hc), O.top1_dense(q, k))


def test_top1_change_rate_counts_queries():
    """The rate is the fraction of Queries whose two argmaxes differ: a cache
    holding the negated Keys flips every Query with a unique positive winner."""
    rng = np.random.default_rng(27)
    d, g = 32, 32
    k = rng.standard_normal((40, d)).astype(np.float32)
    q = rng.standard_normal((20, d))
    hc = O.HeadCache(g, "f32")
    hc.add_epoch(np.zeros((1, d), np.float32), np.ones(1, np.float32), np.zeros((d, 0), np.float32))
    hc.append(k, np.zeros_like(k))
    ref = O.top1_dense(q, k)
    got = O.top1_cached(q, hc)
    expect = float(np.mean(got != ref))
    assert O.top1_change_rate(q, k, hc) == expect
    neg = O.HeadCache(g, "f32")
    neg.add_epoch(np.zeros((1, d), np.float32), np.ones(1, np.float32), np.zeros((d, 0), np.float32))
    neg.append(-k, np.zeros_like(k))
    # the largest logit against -k is the smallest against k: differs unless all equal
    assert O.top1_change_rate(q, k, neg) == 1.0


def test_table1_direction_on_workload_data():
    """The article's attention analysis reports far fewer top-1 changes for
    QuantWM than for QVG. On workload-shaped data the oracle's QuantWM mode
    (QSAC + PSAC) changes fewer top-1 selections than its QVG mode (nearest
    centroid, no compensation) built from the same Keys."""
    w = W.workload("tiny")
    hg = W.HeadGen(w, 0)
    k, v = hg.cache_keys(), hg.cache_values()
    qh = hg.hist_queries()
    q = hg.queries(5, 256).astype(np.float64)
    S, U = O.sensitivity(qh, w.group), O.subspace(qh, w.rank)
    rates = {}
    for name, obj, r in (("quantwm", "qsac", w.rank), ("qvg", "nearest", 0)):
        C = O.build_centroids(k, S, w.n_centroids, w.group, 5, "f32", objective=obj)
        hc = O.HeadCache(w.group, "f32", obj)
        hc.add_epoch(C, S, U[:, :r])
        hc.append(k, v)
        rates[name] = O.top1_change_rate(q, k, hc)
    assert rates["quantwm"] < rates["qvg"]


# ---------------------------------------------------------------- post-rounding error objective

def test_postq_is_the_weighted_error_of_the_stored_record():
    """postq_objective(k, c) is the sensitivity-weighted squared error the
    INT2 record of k would have with centroid c: recomputed in float64 from
    the quantizer's codes and parameters it agrees to float32 rounding, and
    the record that quantize_tokens stores with this rule has exactly the
    smallest such error."""
    rng = np.random.default_rng(31)
    d, g, m, N = 64, 32, 6, 40
    k = rng.standard_normal((N, d)).astype(np.float32) * np.float32(2)
    C = rng.standard_normal((m, d)).astype(np.float32) * np.float32(2)
    S = np.array([1.5, 0.25], np.float32)
    J = O.postq_objective(k, C, S, g)
    for c in range(m):
        r = (k - C[c]).astype(np.float32)
        codes, zp, sc = O.int2_quantize(r, g)
        e = r.astype(np.float64) - O.int2_dequant64(codes, zp, sc, g)
        j64 = ((e ** 2).reshape(N, d // g, g).sum(2) * S.astype(np.float64)).sum(1)
        assert np.all(np.abs(J[:, c] - j64) <= 1e-5 * j64 + 1e-30)
    rec = O.quantize_tokens(k, np.zeros_like(k), C, S, np.zeros((d, 0), np.float32), g, "postq")
    ids = rec["ids"].astype(np.int64)
    assert np.array_equal(ids, np.argmin(J, 1))
    rhat = O.int2_dequant64(rec["kcode"], rec["kzp"], rec["kscale"], g)
    e = (k - C[ids]).astype(np.float64) - rhat
    err = ((e ** 2).reshape(N, d // g, g).sum(2) * S.astype(np.float64)).sum(1)
    assert np.allclose(err, J.min(1), rtol=1e-5)
    # its own optimum: never above the error of the QSAC or nearest choice
    for obj in ("qsac", "nearest"):
        other = O.assign(k, C, S, g, obj)
        assert np.all(J[np.arange(N), ids] <= J[np.arange(N), other])


def test_postq_zero_on_grid_keys_and_half_step_bound():
    """Keys built exactly on the INT2 grid around one centroid have zero
    post-rounding error for it (and that centroid is chosen); every error is
    within the half-step bound sum_G S_G g (step_G / 2)^2."""
    rng = np.random.default_rng(32)
    N, d, g, m = 50, 64, 32, 5
    C = (rng.integers(-40, 40, (m, d)) * 8).astype(np.float32)
    ids = rng.integers(0, m, N)
    zp = (rng.integers(-64, 64, (N, d // g)) / 32).astype(np.float16)
    sc = (rng.integers(1, 32, (N, d // g)) / 64).astype(np.float16)
    codes = rng.integers(0, 4, (N, d)).astype(np.uint8)
    codes.reshape(N, d // g, g)[:, :, 0] = 0
    codes.reshape(N, d // g, g)[:, :, 1] = 3
    k = C[ids] + O.int2_dequant(codes, zp, sc, g)
    S = np.array([1.0, 2.0], np.float32)
    J = O.postq_objective(k, C, S, g)
    assert np.all(J[np.arange(N), ids] == 0)
    assert np.array_equal(O.assign(k, C, S, g, "postq"), ids)
    # half-step bound against each candidate's own quantization step
    for c in range(m):
        _, _, stp = O.int2_quantize((k - C[c]).astype(np.float32), g)
        bound = (S.astype(np.float64) * g * (stp.astype(np.float64) / 2) ** 2).sum(1)
        assert np.all(J[:, c] <= bound * (1 + 1e-5) + 1e-12)


def test_postq_brute_force_argmin_on_tiny_inputs():
    """On tiny random inputs the float32 argmin equals the argmin of the
    float64 error (recomputed from the quantizer's records) wherever the two
    best are not within 1e-6 relative."""
    rng = np.random.default_rng(33)
    checked = 0
    for trial in range(8):
        d, g = 8, 4
        m = int(rng.integers(2, 7))
        N = 40
        k = rng.standard_normal((N, d)).astype(np.float32) * np.float32(2)
        C = rng.standard_normal((m, d)).astype(np.float32) * np.float32(2)
        S = (rng.random(d // g) * 3 + 0.1).astype(np.float32)
        ids = O.assign(k, C, S, g, "postq")
        J64 = np.empty((N, m))
        for c in range(m):
            r = (k - C[c]).astype(np.float32)
            codes, zp, sc = O.int2_quantize(r, g)
            e = r.astype(np.float64) - O.int2_dequant64(codes, zp, sc, g)
            J64[:, c] = ((e ** 2).reshape(N, d // g, g).sum(2) * S.astype(np.float64)).sum(1)
        s = np.sort(J64, 1)
        clear = (s[:, 1] - s[:, 0]) > 1e-6 * s[:, 1]
        assert np.array_equal(ids[clear], np.argmin(J64, 1)[clear])
        checked += int(clear.sum())
    assert checked > 250
