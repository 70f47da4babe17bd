"""GPU parity of the baseline modes and of the top-1 diagnostic, through the
C ABI: QVG's nearest-centroid rule, PSAC switched off (rank 0) and their
combinations, against the CPU oracle's modes; and the top-scoring token per
Query (the article's "Table 1" analysis) for the cache and for full-precision
Keys.

Bar: ids, codes and fp16 parameters bit-exact, coefficients within one fp16
ulp, outputs within 1e-3 of the row's largest magnitude (as for the default
mode). A top-1 index is decided by float32 logits on the GPU and float64 ones
in the oracle, so where two tokens' logits are within the logit tolerance
either is correct: the GPU's choice must score within that tolerance of the
oracle's best, and must equal it wherever the oracle's best two are further
apart."""

import numpy as np
import pytest

import oracle.qwm_oracle as O
import workloads as W
from tests.gpu_helpers import ROW_TOL, compare_records, log, row_rel_err, small, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MODES = [("nearest", 0), ("nearest", None), ("qsac", 0), ("postq", None)]  # None: the workload's rank


def _cache(w, rank, objective, capacity=None, max_q=None, max_build=None):
    from video_world_model_amd import Cache
    return Cache(w.heads, w.head_dim, w.n_centroids, rank, capacity or w.n_kv, dtype=torch_dtype(w.dtype),
                 max_query_tokens=max_q or max(w.n_q, 16), max_build_tokens=max_build or max(w.n_kv, 64),
                 objective=objective)


def _calibrate(w, gens, keys, rank, objective, iters, cal_keys):
    cals = []
    for g, k in zip(gens, keys):
        qh = g.hist_queries()
        S = O.sensitivity(qh, w.group)
        U = O.subspace(qh, rank)
        C = O.build_centroids(k[:cal_keys], S, w.n_centroids, w.group, iters, w.dtype, objective=objective)
        cals.append((C, S, U))
    return cals


def _import(cache, cals, dtype_name, with_S=True):
    C = to_dev([c[0] for c in cals], dtype_name)
    S = torch.from_numpy(np.stack([c[1] for c in cals])).cuda() if with_S else None
    U = torch.from_numpy(np.ascontiguousarray(np.stack([c[2] for c in cals]))).cuda()
    cache.import_calibration(C, S, U)


def _oracle_heads(w, objective, keys, vals, cals):
    hcs = []
    for h in range(w.heads):
        hc = O.HeadCache(w.group, w.dtype, objective)
        hc.add_epoch(*cals[h])
        hc.append(keys[h], vals[h])
        hcs.append(hc)
    return hcs


@pytest.mark.parametrize("objective,rank", MODES)
@pytest.mark.parametrize("name,heads,n_kv,n_q,mask", [
    ("tiny", 1, 1024, 16, "none"),
    ("video_chunk", 3, 2500, 300, "full"),
])
def test_mode_quantize_and_attend(objective, rank, name, heads, n_kv, n_q, mask):
    w = small(W.workload(name), heads=heads, n_kv=n_kv, n_q=n_q, n_self=n_q if mask != "none" else 0)
    r = w.rank if rank is None else rank
    log(f"[mode parity] {name} objective={objective} rank={r} H={heads} n_kv={n_kv} n_q={n_q} mask={mask}")
    gens = [W.HeadGen(w, h) for h in range(heads)]
    keys = [g.keys(0, n_kv) for g in gens]
    vals = [g.values(0, n_kv) for g in gens]
    cals = _calibrate(w, gens, keys, r, objective, 2, min(n_kv, 880))
    cache = _cache(w, r, objective)
    _import(cache, cals, w.dtype)
    cache.quantize_append(to_dev(keys, w.dtype), to_dev(vals, w.dtype))
    dec = cache.decode_export(cache.export().cpu().numpy(), n_kv)
    for h in range(heads):
        rec = O.quantize_tokens(keys[h], vals[h], *cals[h], w.group, objective)
        assert rec["coef"].shape == (n_kv, r)
        compare_records(dec, h, rec)
    q = [g.current_queries()[:n_q] for g in gens]
    ks = vs = None
    if mask != "none":
        ks = [g.keys(n_kv, n_kv + n_q) for g in gens]
        vs = [g.values(n_kv, n_kv + n_q) for g in gens]
        out = cache.attend(to_dev(q, w.dtype), to_dev(ks, w.dtype), to_dev(vs, w.dtype), mask=mask)
    else:
        out = cache.attend(to_dev(q, w.dtype))
    out = out.cpu().numpy()
    hcs = _oracle_heads(w, objective, keys, vals, cals)
    worst = 0.0
    for h in range(heads):
        ref = O.attend(q[h], hcs[h], None if ks is None else ks[h], None if vs is None else vs[h], mask=mask)
        e = row_rel_err(out[h], ref)
        worst = max(worst, float(e.max()))
        assert e.max() <= ROW_TOL, f"head {h}: row error {e.max():.3e}"
    log(f"  worst row error {worst:.3e}")


def test_nearest_rank0_without_sensitivity():
    """QVG needs no historical Queries: a calibration imported without S_G
    stores zeros and quantizes exactly like one with S_G."""
    w = small(W.workload("video_chunk"), heads=2, n_kv=700)
    gens = [W.HeadGen(w, h) for h in range(2)]
    keys = [g.keys(0, 700) for g in gens]
    vals = [g.values(0, 700) for g in gens]
    cals = _calibrate(w, gens, keys, 0, "nearest", 1, 700)
    a = _cache(w, 0, "nearest")
    _import(a, cals, w.dtype, with_S=True)
    b = _cache(w, 0, "nearest")
    _import(b, cals, w.dtype, with_S=False)
    for c in (a, b):
        c.quantize_append(to_dev(keys, w.dtype), to_dev(vals, w.dtype))
    assert np.array_equal(a.export().cpu().numpy(), b.export().cpu().numpy())
    _, S, _ = b.export_calibration(0)
    assert torch.count_nonzero(S).item() == 0


@pytest.mark.parametrize("name,heads,n_keys,iters", [("tiny", 1, 1024, 4), ("video_chunk", 2, 1200, 3)])
def test_postq_build(name, heads, n_keys, iters):
    """GPU k-means with the post-rounding error rule reaches the oracle
    build's mean error within 1%."""
    w = small(W.workload(name), heads=heads)
    log(f"[postq build] {name} H={heads} n_keys={n_keys} iters={iters}")
    gens = [W.HeadGen(w, h) for h in range(heads)]
    keys = [g.keys(0, n_keys) for g in gens]
    qh = [g.hist_queries() for g in gens]
    cache = _cache(w, w.rank, "postq", max_build=n_keys)
    cache.build_subspace(to_dev(qh, w.dtype))
    cache.build_centroids(to_dev(keys, w.dtype), iters)
    C, S, _ = (t.cpu() for t in cache.export_calibration(0))
    C = C.float().numpy()
    S = S.numpy()
    for h in range(heads):
        Co = O.build_centroids(keys[h], S[h], w.n_centroids, w.group, iters, w.dtype, objective="postq")
        jg = O.mean_objective(keys[h], C[h], S[h], w.group, "postq")
        jo = O.mean_objective(keys[h], Co, S[h], w.group, "postq")
        log(f"  head {h}: mean error gpu {jg:.6g} oracle {jo:.6g} identical {np.array_equal(C[h], Co)}")
        assert abs(jg - jo) <= 0.01 * jo


@pytest.mark.parametrize("name,heads,n_keys,iters,with_subspace", [
    ("tiny", 1, 1024, 10, False),
    ("video_chunk", 3, 1760, 4, True),
    ("video_chunk", 2, 4000, 4, False),  # 64 centroids: the full pass every iteration
    ("wm_layer", 2, 9000, 5, False),  # 256 centroids, >= 32 Keys each: the pruned assignment
])
def test_nearest_build(name, heads, n_keys, iters, with_subspace):
    """GPU k-means with the nearest-centroid rule (QVG, rank 0) reaches the
    oracle build's mean squared distance within 1%; it runs with or without a
    staged subspace."""
    w = small(W.workload(name), heads=heads)
    log(f"[nearest build] {name} H={heads} n_keys={n_keys} iters={iters}")
    gens = [W.HeadGen(w, h) for h in range(heads)]
    keys = [g.keys(0, n_keys) for g in gens]
    cache = _cache(w, 0, "nearest", max_build=n_keys)
    if with_subspace:
        cache.build_subspace(to_dev([g.hist_queries() for g in gens], w.dtype))
    cache.build_centroids(to_dev(keys, w.dtype), iters)
    C = cache.export_calibration(0)[0].cpu().float().numpy()
    zero = np.zeros(w.head_dim // 32, np.float32)
    for h in range(heads):
        Co = O.build_centroids(keys[h], zero, w.n_centroids, w.group, iters, w.dtype, objective="nearest")
        jg = O.mean_objective(keys[h], C[h], zero, w.group, "nearest")
        jo = O.mean_objective(keys[h], Co, zero, w.group, "nearest")
        log(f"  head {h}: mean distance gpu {jg:.6g} oracle {jo:.6g} identical {np.array_equal(C[h], Co)}")
        assert abs(jg - jo) <= 0.01 * jo
        if w.dtype == "bf16":
            assert np.array_equal(C[h], Co)  # exact float64 sums, bit-exact ids


def _check_top1(got, logits64, tol_rel):
    """got [n_q] indices, logits64 [n_q][n] oracle logits. Returns (#rows where
    the oracle's best is clear, #rows equal)."""
    n_q = logits64.shape[0]
    rows = np.arange(n_q)
    best = logits64.max(1)
    tol = tol_rel * np.abs(logits64).max(1)
    assert np.all((got >= 0) & (got < logits64.shape[1]))
    assert np.all(logits64[rows, got] >= best - tol), "a top-1 index scores below the oracle's best"
    s = np.sort(logits64, 1)
    clear = (s[:, -1] - s[:, -2]) > tol
    ref = np.argmax(logits64, 1)
    assert np.array_equal(got[clear], ref[clear])
    return int(clear.sum()), int((got == ref).sum())


@pytest.mark.parametrize("objective,rank", [("qsac", None), ("nearest", 0)])
@pytest.mark.parametrize("name,heads,n_kv,n_q", [("tiny", 1, 1024, 16), ("video_chunk", 2, 3333, 150)])
def test_top1_matches_oracle(objective, rank, name, heads, n_kv, n_q):
    w = small(W.workload(name), heads=heads, n_kv=n_kv, n_q=n_q)
    r = w.rank if rank is None else rank
    log(f"[top1] {name} objective={objective} rank={r} H={heads} n_kv={n_kv} n_q={n_q}")
    gens = [W.HeadGen(w, h) for h in range(heads)]
    keys = [g.keys(0, n_kv) for g in gens]
    vals = [g.values(0, n_kv) for g in gens]
    cals = _calibrate(w, gens, keys, r, objective, 2, min(n_kv, 880))
    cache = _cache(w, r, objective, max_q=n_q)
    _import(cache, cals, w.dtype)
    kd = to_dev(keys, w.dtype)
    cache.quantize_append(kd, to_dev(vals, w.dtype))
    q = [g.current_queries()[:n_q] for g in gens]
    qd = to_dev(q, w.dtype)
    t_cache = cache.attend_top1(qd).cpu().numpy()
    t_ref = cache.attend_top1(qd, kd).cpu().numpy()
    hcs = _oracle_heads(w, objective, keys, vals, cals)
    for h in range(heads):
        ell = O.cache_logits(q[h], hcs[h], 1.0)
        full = np.asarray(q[h], np.float64) @ np.asarray(keys[h], np.float64).T
        c1, e1 = _check_top1(t_cache[h], ell, 2 * ROW_TOL)
        c2, e2 = _check_top1(t_ref[h], full, ROW_TOL / 10)
        rate_gpu = float(np.mean(t_cache[h] != t_ref[h]))
        rate_oracle = O.top1_change_rate(q[h], keys[h], hcs[h])
        log(f"  head {h}: cache top-1 equal {e1}/{n_q} (clear {c1}); full-precision equal {e2}/{n_q} "
            f"(clear {c2}); change rate gpu {rate_gpu:.3f} oracle {rate_oracle:.3f}")
        assert abs(rate_gpu - rate_oracle) <= (2 * n_q - c1 - c2) / n_q + 1e-12


def _tie_case(gens, n_ref):
    """Queries that all point along one sign pattern and a reference whose rows
    100 and n_ref - 101 are the same dominant Key 256 * sign(q0): every Query's
    largest logit is shared by those two rows (all values bf16-exact)."""
    qs, refs = [], []
    for g in gens:
        q0 = g.current_queries()[0].astype(np.float64)
        q = np.stack([q0 * (1.0 + i / 40.0) for i in range(40)]).astype(np.float32)
        qs.append(W.round_to_bf16(q))
        k = g.keys(64, 64 + n_ref).copy()
        win = (256.0 * np.sign(q0)).astype(np.float32)
        k[100] = win
        k[n_ref - 101] = win
        refs.append(k)
    return qs, refs


def test_top1_ties_and_ragged_reference():
    """Equal logits go to the smallest token index, across tiles and splits,
    with a ragged last tile (3001 Keys)."""
    w = small(W.workload("video_chunk"), heads=2, n_kv=64, n_q=40)
    gens = [W.HeadGen(w, h) for h in range(2)]
    keys = [g.keys(0, 64) for g in gens]
    vals = [g.values(0, 64) for g in gens]
    cals = _calibrate(w, gens, keys, w.rank, "qsac", 1, 64)
    cache = _cache(w, w.rank, "qsac", max_q=40)
    _import(cache, cals, w.dtype)
    cache.quantize_append(to_dev(keys, w.dtype), to_dev(vals, w.dtype))
    q, ref = _tie_case(gens, 3001)
    t = cache.attend_top1(to_dev(q, w.dtype), to_dev(ref, w.dtype)).cpu().numpy()
    for h in range(2):
        full = np.asarray(q[h], np.float64) @ np.asarray(ref[h], np.float64).T
        assert np.all(np.argmax(full, 1) == 100)
        assert np.all(t[h] == 100), t[h]
