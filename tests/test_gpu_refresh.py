"""GPU parity of the in-stream calibration refresh (roboind.com article,
"Step 1" and "Step 2": centroids and the PSAC basis come from historical
Queries and recent Keys, so a streaming cache is recalibrated as it grows;
fugumt.com abstract: strictly causal, tokens already stored keep their
epoch).

Every epoch's calibration is built ON THE GPU (build_subspace +
build_centroids) at its boundary. Bars:
  * the GPU calibration against the oracle's own build from the same inputs:
    S_G bit-exact, projector within 1e-4, bf16 centroids bit-identical;
  * every record against the oracle quantizing with the calibration the GPU
    exported for that token's epoch: bit-exact (1 fp16 ulp for PSAC
    coefficients), epoch tags equal;
  * attention over all epochs within 1e-3 of the row maximum, on the prefill
    path (96 Queries) and the decode path (16 Queries).
The sequence also truncates into an earlier epoch and appends again (the
earlier epoch's calibration becomes current), and then repeats the
streaming bench's refresh: truncate to an epoch boundary and rebuild, which
replaces the epoch that now holds no token."""

import numpy as np
import pytest

import oracle.qwm_oracle as O
import workloads as W
from tests.gpu_helpers import ROW_TOL, compare_records, log, row_rel_err, small, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

LENS = (1000, 1777, 640)   # ragged epochs
BUILD = (800, 700, 640)    # Keys each epoch's centroids are built from (its first tokens)
N_HIST = 1500
ITERS = 3


def _check_calibration(w, C, S, U, qh, keys):
    """GPU calibration of one head against the oracle's build from the same inputs."""
    So = O.sensitivity(qh, w.group)
    assert np.array_equal(S, So), (S, So)
    Uo = O.subspace(qh, w.rank)
    P1 = U.astype(np.float64) @ U.astype(np.float64).T
    P2 = Uo.astype(np.float64) @ Uo.astype(np.float64).T
    perr = np.linalg.norm(P1 - P2) / np.linalg.norm(P2)
    assert perr < 1e-4, perr
    Co = O.build_centroids(keys, So, w.n_centroids, w.group, ITERS, w.dtype)
    assert np.array_equal(C, Co), "GPU centroids differ from the oracle build"
    return perr


def _export_cal(cache, epoch):
    C, S, U = (t.cpu() for t in cache.export_calibration(epoch))
    return C.float().numpy(), S.numpy(), U.numpy()


def _compare_all(cache, hcs, n):
    dec = cache.decode_export(cache.export().cpu().numpy(), n)
    flips = 0
    for h, hc in enumerate(hcs):
        assert hc.length == n
        for start, rec in hc.records:
            flips += compare_records(dec, h, rec, start)
        assert np.array_equal(dec["epoch"][h], hc.field("epoch"))
    return flips


def _attend_check(cache, hcs, gens, w, nq):
    q = [g.current_queries()[:nq] for g in gens]
    out = cache.attend(to_dev(q, w.dtype)).cpu().numpy()
    worst = 0.0
    for h, hc in enumerate(hcs):
        err = row_rel_err(out[h], O.attend(q[h], hc)).max()
        worst = max(worst, err)
    assert worst <= ROW_TOL, worst
    return worst


def test_refresh_in_stream_matches_oracle():
    from video_world_model_amd import Cache
    w = small(W.workload("streaming"), heads=2, n_q=96)
    H = w.heads
    gens = [W.HeadGen(w, h) for h in range(H)]
    total = sum(LENS)
    cache = Cache(H, w.head_dim, w.n_centroids, w.rank, total, dtype=torch.bfloat16, max_epochs=3,
                  max_query_tokens=96, max_build_tokens=max(BUILD))
    starts = np.cumsum((0,) + LENS)
    cals = []  # per epoch: per head (C, S, U) exported from the GPU
    for e, n in enumerate(LENS):
        t0 = int(starts[e])
        log(f"[refresh] epoch {e}: tokens {t0}..{t0 + n}, GPU build from {BUILD[e]} Keys and {N_HIST} Queries")
        qh = [g.queries(W.Q_HIST + e, N_HIST) for g in gens]
        keys = [g.keys(t0, t0 + n) for g in gens]
        vals = [g.values(t0, t0 + n) for g in gens]
        cache.build_subspace(to_dev(qh, w.dtype))
        cache.build_centroids(to_dev([k[:BUILD[e]] for k in keys], w.dtype), ITERS)
        half = n // 2 + 3  # two appends per epoch, a ragged split
        cache.quantize_append(to_dev([k[:half] for k in keys], w.dtype), to_dev([v[:half] for v in vals], w.dtype))
        cache.quantize_append(to_dev([k[half:] for k in keys], w.dtype), to_dev([v[half:] for v in vals], w.dtype))
        cal = [tuple(x[h] for x in _export_cal(cache, e)) for h in range(H)]
        for h in range(H):
            perr = _check_calibration(w, *cal[h], qh[h], keys[h][:BUILD[e]])
            log(f"  head {h}: S bit-exact, projector error {perr:.1e}, centroids bit-identical")
        cals.append(cal)
    assert cache.epochs() == 3 and cache.length() == total

    def oracle_caches(epochs):
        """Oracle head caches: for each (calibrations, t0, t1) the tokens of
        [t0, t1) appended under that epoch's exported calibration."""
        hcs = [O.HeadCache(w.group, w.dtype) for _ in range(H)]
        for cal, t0, t1 in epochs:
            for h in range(H):
                hcs[h].add_epoch(*cal[h])
                hcs[h].append(gens[h].keys(t0, t1), gens[h].values(t0, t1))
        return hcs

    hcs = oracle_caches([(cals[e], int(starts[e]), int(starts[e + 1])) for e in range(3)])
    flips = _compare_all(cache, hcs, total)
    log(f"  3-epoch records bit-exact ({flips} coefficient one-ulp differences)")
    log(f"  prefill attention worst row error {_attend_check(cache, hcs, gens, w, 96):.2e}")
    log(f"  decode attention worst row error {_attend_check(cache, hcs, gens, w, 16):.2e}")

    # truncate into epoch 1: epoch 2 is dropped, epoch 1's calibration is
    # current again; append the rest of epoch 1 and compare
    cut = int(starts[1]) + 611
    cache.truncate(cut)
    assert cache.epochs() == 2 and cache.length() == cut
    e1 = int(starts[2])
    cache.quantize_append(to_dev([g.keys(cut, e1) for g in gens], w.dtype),
                          to_dev([g.values(cut, e1) for g in gens], w.dtype))
    hcs = oracle_caches([(cals[0], 0, int(starts[1])), (cals[1], int(starts[1]), e1)])
    _compare_all(cache, hcs, e1)
    log(f"  truncate into epoch 1 at {cut} and re-append: records bit-exact")

    # the streaming refresh: the epoch started at the boundary holds no token
    # after this truncate and is replaced by the rebuild. The historical
    # Queries are a temporary that is freed and overwritten before the
    # centroid build (every read of it is on the cache stream).
    cache.quantize_append(to_dev([g.keys(e1, e1 + 100) for g in gens], w.dtype),
                          to_dev([g.values(e1, e1 + 100) for g in gens], w.dtype))
    assert cache.epochs() == 2
    cache.truncate(e1)
    qh2 = [g.queries(W.Q_HIST + 7, N_HIST) for g in gens]
    keys2 = [g.keys(e1, e1 + LENS[2]) for g in gens]
    cache.build_subspace(to_dev(qh2, w.dtype))  # the device copy is released here
    junk = torch.full((H, N_HIST, w.head_dim), 3.0e3, dtype=torch.bfloat16, device="cuda")
    cache.build_centroids(to_dev([k[:BUILD[2]] for k in keys2], w.dtype), ITERS)
    del junk
    assert cache.epochs() == 3
    cache.quantize_append(to_dev(keys2, w.dtype), to_dev([g.values(e1, e1 + LENS[2]) for g in gens], w.dtype))
    cal2 = [tuple(x[h] for x in _export_cal(cache, 2)) for h in range(H)]
    for h in range(H):
        _check_calibration(w, *cal2[h], qh2[h], keys2[h][:BUILD[2]])
    hcs = oracle_caches([(cals[0], 0, int(starts[1])), (cals[1], int(starts[1]), e1), (cal2, e1, total)])
    _compare_all(cache, hcs, total)
    log(f"  truncate to the boundary {e1} and rebuild: calibration matches the oracle build, records bit-exact")
    log(f"  prefill attention worst row error {_attend_check(cache, hcs, gens, w, 96):.2e}")
    log(f"  decode attention worst row error {_attend_check(cache, hcs, gens, w, 16):.2e}")
