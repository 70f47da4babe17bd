"""Pins of the oracle's multi-epoch cache (``HeadCache`` with several
calibrations): each token keeps the centroids, sensitivity and PSAC basis of
the epoch it was appended in, and an epoch that holds no token yet is
replaced by the next one (roboind.com article, "Step 1" and "Step 2":
calibration comes from historical Queries, so it is refreshed as the video
goes on; the fugumt.com abstract: strictly causal, so tokens already stored
are never re-quantized).

The references are independent of the multi-epoch code: single-epoch caches
(whose path the other pins fix) built side by side, the raw Keys themselves
at full PSAC rank, and the log-sum-exp merge of attention over disjoint
token sets."""

import numpy as np

import oracle.qwm_oracle as O

D, G, M = 64, 32, 4
LENS = (37, 50, 29)  # ragged epochs


def _epoch(rng, r, n):
    """One epoch's calibration (distinct per epoch) and its tokens."""
    C = (rng.standard_normal((M, D)) * 2.0).astype(np.float32)
    S = rng.uniform(0.5, 2.0, D // G).astype(np.float32)
    U = np.linalg.qr(rng.standard_normal((D, D)))[0][:, :r].astype(np.float32)
    k = (C[rng.integers(0, M, n)] + 0.4 * rng.standard_normal((n, D))).astype(np.float32)
    v = rng.standard_normal((n, D)).astype(np.float32)
    return C, S, U, k, v


def _caches(r, seed=7):
    rng = np.random.default_rng(seed)
    eps = [_epoch(rng, r, n) for n in LENS]
    multi = O.HeadCache(G, "f32")
    singles = []
    for C, S, U, k, v in eps:
        multi.add_epoch(C, S, U)
        multi.append(k, v)
        one = O.HeadCache(G, "f32")
        one.add_epoch(C, S, U)
        one.append(k, v)
        singles.append(one)
    q = (rng.standard_normal((9, D)) * 1.5).astype(np.float32)
    return eps, multi, singles, q


def test_records_and_dequantized_keys_follow_their_epoch():
    """Every token's stored record, and its dequantized Key c_id + zp + code *
    step, equal those of a one-epoch cache holding that epoch's calibration."""
    _, multi, singles, _ = _caches(r=8)
    for f in ("ids", "kcode", "vcode", "kzp", "kscale", "vzp", "vscale", "coef"):
        got = multi.field(f)
        ref = np.concatenate([one.field(f) for one in singles])
        assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), f
    assert np.array_equal(multi.field("epoch"), np.repeat(np.arange(3), LENS))
    assert np.array_equal(multi.khat64(), np.concatenate([one.khat64() for one in singles]))


def test_logits_are_the_single_epoch_logits_side_by_side():
    """Compensated logits over a three-epoch cache are the three one-epoch
    caches' logits concatenated: each token's PSAC term uses its own epoch's
    basis."""
    _, multi, singles, q = _caches(r=8)
    got = O.cache_logits(q, multi, 0.125)
    ref = np.concatenate([O.cache_logits(q, one, 0.125) for one in singles], axis=1)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_attention_is_the_lse_merge_of_the_epochs():
    """Softmax attention over the whole cache equals the log-sum-exp merge of
    attention over each epoch's tokens alone."""
    _, multi, singles, q = _caches(r=8)
    scale = 1.0 / np.sqrt(D)
    got = O.attend(q, multi)
    lse = []
    outs = []
    for one in singles:
        ell = O.cache_logits(q, one, scale)
        mx = ell.max(axis=1, keepdims=True)
        lse.append((mx + np.log(np.exp(ell - mx).sum(axis=1, keepdims=True)))[:, 0])
        outs.append(O.attend(q, one))
    lse = np.stack(lse)  # [epochs][Nq]
    L = lse.max(axis=0) + np.log(np.exp(lse - lse.max(axis=0)).sum(axis=0))
    ref = sum(np.exp(lse[e] - L)[:, None] * outs[e] for e in range(3))
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_full_rank_restores_every_epochs_exact_logits():
    """At r = d every epoch's basis is a different orthogonal matrix U_e with
    U_e U_e^T = I, so q . khat + (q U_e) . (U_e^T e) = q . k exactly for the
    raw Key k, up to the fp16 rounding of the coefficients: |error| <=
    sum_k |(q U_e)_k| ulp(coef_k) / 2. A basis of the wrong epoch breaks this
    by far more than the bound."""
    eps, multi, _, q = _caches(r=D)
    got = O.cache_logits(q, multi, 1.0)
    coef = multi.field("coef").astype(np.float64)
    half_ulp = np.spacing(np.abs(multi.field("coef"))).astype(np.float64) / 2
    ep = multi.field("epoch")
    t0 = 0
    worst_rel = 0.0
    for e, (C, S, U, k, v) in enumerate(eps):
        sl = slice(t0, t0 + len(k))
        exact = q.astype(np.float64) @ k.astype(np.float64).T
        qU = np.abs(q.astype(np.float64) @ U.astype(np.float64))
        bound = qU @ half_ulp[sl].T + 1e-9 * np.abs(exact).max()
        err = np.abs(got[:, sl] - exact)
        assert np.all(err <= bound), f"epoch {e}: {np.max(err - bound)} beyond the fp16 bound"
        worst_rel = max(worst_rel, float((err / np.maximum(bound, 1e-300)).max()))
        assert np.all(ep[sl] == e)
        t0 += len(k)
    # the other epochs' bases do not restore the logits: the pin can fail
    C, S, U, k, v = eps[1]
    U_wrong = eps[2][2].astype(np.float64)
    sl = slice(LENS[0], LENS[0] + LENS[1])
    khat = multi.khat64()[sl]
    wrong = q.astype(np.float64) @ khat.T + (q.astype(np.float64) @ U_wrong) @ coef[sl].T
    exact = q.astype(np.float64) @ k.astype(np.float64).T
    assert np.abs(wrong - exact).max() > 100 * np.abs(got[:, sl] - exact).max()


def test_an_empty_epoch_is_replaced():
    """A calibration committed while the last epoch holds no token replaces
    that epoch: the cache then equals one that only ever had the second
    calibration; after tokens arrive a new calibration opens a new epoch."""
    rng = np.random.default_rng(11)
    Ca, Sa, Ua, ka, va = _epoch(rng, 8, 20)
    Cb, Sb, Ub, kb, vb = _epoch(rng, 8, 20)
    Cc, Sc, Uc, kc, vc = _epoch(rng, 8, 20)
    h = O.HeadCache(G, "f32")
    h.add_epoch(Ca, Sa, Ua)
    h.add_epoch(Cb, Sb, Ub)  # replaces the empty first epoch
    assert len(h.epochs) == 1
    h.append(kb, vb)
    ref = O.HeadCache(G, "f32")
    ref.add_epoch(Cb, Sb, Ub)
    ref.append(kb, vb)
    for f in ("ids", "kcode", "kzp", "kscale", "coef"):
        assert np.array_equal(h.field(f).view(np.uint8), ref.field(f).view(np.uint8)), f
    h.add_epoch(Ca, Sa, Ua)
    h.add_epoch(Cc, Sc, Uc)  # the Ca epoch at position 20 is still empty: replaced
    assert len(h.epochs) == 2 and h.epochs[1][0] == 20
    h.append(kc, vc)
    one = O.HeadCache(G, "f32")
    one.add_epoch(Cc, Sc, Uc)
    one.append(kc, vc)
    assert np.array_equal(h.field("ids")[20:], one.field("ids"))
    assert np.array_equal(h.field("epoch"), np.repeat([0, 1], 20))
    q = rng.standard_normal((5, D)).astype(np.float32)
    np.testing.assert_allclose(O.cache_logits(q, h, 1.0)[:, 20:], O.cache_logits(q, one, 1.0), rtol=1e-12,
                               atol=1e-12)
