"""GPU parity of decode-shaped attention (at most 48 Queries per head over
bf16 Keys, no self segment), which runs on its own kernel: the 2-bit codes
are the MFMA operand, q . C comes from a per-Query table, one wave per
workgroup over many splits of the cache. Same bar as every attention test:
outputs within 1e-3 of the row's largest magnitude against the oracle."""

import numpy as np
import pytest

import oracle.qwm_oracle as O
import workloads as W
from tests.gpu_helpers import ROW_TOL, import_calibration, log, oracle_calibration, row_rel_err, small, to_dev, \
    torch_dtype

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _cache(w, rank=None, capacity=None, max_epochs=1, max_q=64, objective="qsac"):
    from video_world_model_amd import Cache
    return Cache(w.heads, w.head_dim, w.n_centroids, w.rank if rank is None else rank, capacity or w.n_kv,
                 dtype=torch_dtype(w.dtype), max_epochs=max_epochs, max_query_tokens=max_q,
                 max_build_tokens=max(w.n_kv, 64), objective=objective)


@pytest.mark.parametrize("n_q", [1, 5, 16, 17, 33, 48])
def test_decode_matches_oracle(n_q):
    w = small(W.workload("video_chunk"), heads=3, n_kv=3000, n_q=n_q)
    log(f"[decode] video_chunk H=3 n_kv=3000 n_q={n_q}")
    gens = [W.HeadGen(w, h) for h in range(3)]
    keys = [g.keys(0, 3000) for g in gens]
    vals = [g.values(0, 3000) for g in gens]
    cals = [oracle_calibration(w, g, k[:880], g.hist_queries(), 2) for g, k in zip(gens, keys)]
    cache = _cache(w)
    import_calibration(cache, cals, w.dtype)
    cache.quantize_append(to_dev(keys, w.dtype), to_dev(vals, w.dtype))
    q = [g.current_queries()[:n_q] for g in gens]
    out = cache.attend(to_dev(q, w.dtype)).cpu().numpy()
    worst = 0.0
    for h in range(3):
        hc = O.HeadCache(w.group, w.dtype)
        hc.add_epoch(*cals[h])
        hc.append(keys[h], vals[h])
        e = row_rel_err(out[h], O.attend(q[h], hc))
        worst = max(worst, float(e.max()))
        assert e.max() <= ROW_TOL, f"head {h}: row error {e.max():.3e}"
    log(f"  worst row error {worst:.3e}")


@pytest.mark.parametrize("objective,rank,scale", [("nearest", 0, None), ("qsac", 4, -0.05), ("qsac", 16, 0.2)])
def test_decode_modes_epochs_and_scale(objective, rank, scale):
    """Three epochs of ragged lengths, both centroid rules, rank 0 to 16, and
    a negative softmax scale."""
    w = small(W.workload("video_chunk"), heads=2, n_q=24)
    lens = [700, 1301, 419]
    log(f"[decode epochs] objective={objective} rank={rank} scale={scale} lens={lens}")
    gens = [W.HeadGen(w, h) for h in range(2)]
    cache = _cache(w, rank=rank, capacity=sum(lens), max_epochs=3, objective=objective)
    hcs = [O.HeadCache(w.group, w.dtype, objective) for _ in range(2)]
    t = 0
    for e, n in enumerate(lens):
        keys = [g.keys(t, t + n) for g in gens]
        vals = [g.values(t, t + n) for g in gens]
        cals = []
        for g, k in zip(gens, keys):
            qh = g.hist_queries(e)
            S = O.sensitivity(qh, w.group)
            cals.append((O.build_centroids(k[:300], S, w.n_centroids, w.group, 1, w.dtype, objective=objective), S,
                         O.subspace(qh, rank)))
        import_calibration(cache, cals, w.dtype)
        cache.quantize_append(to_dev(keys, w.dtype), to_dev(vals, w.dtype))
        for h in range(2):
            hcs[h].add_epoch(*cals[h])
            hcs[h].append(keys[h], vals[h])
        t += n
    q = [g.current_queries()[:24] for g in gens]
    out = cache.attend(to_dev(q, w.dtype), scale=scale).cpu().numpy()
    for h in range(2):
        e = row_rel_err(out[h], O.attend(q[h], hcs[h], scale=scale))
        log(f"  head {h}: worst row error {e.max():.3e}")
        assert e.max() <= ROW_TOL
