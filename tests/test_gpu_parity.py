"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bar: centroid ids, INT2 codes and fp16 zero-points/steps bit-exact given the
same (imported) calibration; PSAC coefficients within one fp16 ulp (float64
dot products summed in a different order may round differently); logits and
attention outputs within 1e-3 of the row's largest magnitude."""

import numpy as np
import pytest

import oracle.qwm_oracle as O
import workloads as W
from tests.gpu_helpers import (ROW_TOL, compare_records, import_calibration, log, oracle_calibration, row_rel_err,
                               small, to_dev, torch_dtype)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _cache(w, capacity=None, max_epochs=1, max_q=None, max_build=None):
    from video_world_model_amd import Cache
    return Cache(w.heads, w.head_dim, w.n_centroids, w.rank, capacity or w.n_kv, dtype=torch_dtype(w.dtype),
                 max_epochs=max_epochs, max_query_tokens=max_q or max(w.n_q, 16),
                 max_build_tokens=max_build or max(w.n_kv, 64))


def _setup(w, n_kv, cal_keys, iters, seed=0):
    """Generator arrays + oracle calibration + oracle head caches for heads 0..H-1."""
    gens = [W.HeadGen(w, h, seed) for h in range(w.heads)]
    keys = [g.keys(0, n_kv) for g in gens]
    vals = [g.values(0, n_kv) for g in gens]
    cals = [oracle_calibration(w, g, k[:cal_keys], g.hist_queries(), iters) for g, k in zip(gens, keys)]
    return gens, keys, vals, cals


# (seeds 1 and 2: the same shapes from other generator streams)
@pytest.mark.parametrize("name,heads,n_kv,cal_keys,iters,seed", [
    ("tiny", 1, 1024, 1024, 10, 0),
    ("video_chunk", 12, 7040, 880, 2, 0),
    ("tiny", 1, 1024, 1024, 10, 1),
    ("video_chunk", 2, 2000, 880, 2, 2),
])
def test_quantize_bit_exact(name, heads, n_kv, cal_keys, iters, seed):
    w = small(W.workload(name), heads=heads, n_kv=n_kv)
    log(f"[quantize parity] {name} H={heads} n={n_kv} seed={seed}")
    gens, keys, vals, cals = _setup(w, n_kv, cal_keys, iters, seed)
    cache = _cache(w)
    import_calibration(cache, cals, w.dtype)
    cache.quantize_append(to_dev(keys, w.dtype), to_dev(vals, w.dtype))
    dec = cache.decode_export(cache.export().cpu().numpy(), n_kv)
    flips = 0
    for h in range(heads):
        rec = O.quantize_tokens(keys[h], vals[h], *cals[h], w.group)
        flips += compare_records(dec, h, rec)
    assert np.all(dec["epoch"] == 0)
    log(f"  coef fp16 one-ulp differences: {flips} of {heads * n_kv * w.rank}")



def _tie_rows(rng, n, d, dtype):
    """Rows whose 32-channel groups have min z and max z + 3s with s a power of
    two, so zero-point = z and step = s exactly, and whose other channels sit
    at z + (k + 1/2) s (ties: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2) or one ulp of the
    input dtype to either side of them."""
    ties = np.array([0.5, 1.5, 2.5], np.float32)
    rows = np.empty((n, d), np.float32)
    for t in range(n):
        for g0 in range(0, d, 32):
            s = np.float32(2.0) ** rng.integers(-6, 5)
            z = np.float32(rng.choice([0.0, -1.25, 0.75, -3.0]))
            q = ties[rng.integers(0, 3, 32)]
            x = (z + q * s).astype(np.float32)
            step = rng.integers(-1, 2, 32) * (x != 0)  # one ulp down, none, up (zeros stay)
            if dtype == "bf16":
                xb = W.bf16_bits(W.round_to_bf16(x)).astype(np.int32) + np.where(x < 0, -1, 1) * step
                x = (xb.astype(np.uint32) << 16).view(np.float32)
            else:
                x = np.where(step > 0, np.nextafter(x, np.float32(np.inf)),
                             np.where(step < 0, np.nextafter(x, np.float32(-np.inf)), x)).astype(np.float32)
            x[0], x[1] = z, z + 3 * s
            rows[t, g0:g0 + 32] = x
    if dtype == "bf16":  # the values the device receives
        rows = W.round_to_bf16(rows)
    assert np.all(np.isfinite(rows))
    return rows


@pytest.mark.parametrize("name", ["tiny", "video_chunk"])
def test_quantize_half_integer_ties(name):
    """INT2 codes of quotients at and one ulp around 0.5, 1.5, 2.5: the
    kernels round the reciprocal product and fall back to the correctly
    rounded divide next to a half-integer; the codes must be the oracle's."""
    w = small(W.workload(name), heads=1, n_kv=256)
    rng = np.random.default_rng(7)
    g = W.HeadGen(w, 0)
    keys = [_tie_rows(rng, 256, w.head_dim, w.dtype)]
    vals = [_tie_rows(rng, 256, w.head_dim, w.dtype)]
    C = np.zeros((w.n_centroids, w.head_dim), np.float32)  # residual = Key; every id ties to 0
    S = O.sensitivity(g.hist_queries(), w.group)
    U = O.subspace(g.hist_queries(), w.rank)
    cals = [(C, S, U)]
    cache = _cache(w)
    import_calibration(cache, cals, w.dtype)
    cache.quantize_append(to_dev(keys, w.dtype), to_dev(vals, w.dtype))
    dec = cache.decode_export(cache.export().cpu().numpy(), 256)
    rec = O.quantize_tokens(keys[0], vals[0], C, S, U, w.group)
    compare_records(dec, 0, rec)
    log(f"  {name}: codes equal the oracle's over {256 * w.head_dim} Key and Value channels")

def _degenerate_rows(rng, n, d, dtype, C):
    """Rows whose 32-channel groups are edge cases of the quantizer: constant
    groups (zero range: step 0, codes 0), tiny magnitudes (fp16 zero-points
    and steps in the subnormal range), one outlier among zeros, signed zeros,
    large magnitudes (steps near 10^4), plain values, and whole rows equal to
    a centroid (zero residual)."""
    rows = np.empty((n, d), np.float32)
    for t in range(n):
        if t % 7 == 6:
            rows[t] = C[rng.integers(0, C.shape[0])]
            continue
        for g0 in range(0, d, 32):
            kind = rng.integers(0, 6)
            if kind == 0:
                x = np.full(32, rng.choice([0.0, -1.5, 0.3125, 7.0]), np.float32)
            elif kind == 1:
                x = (rng.standard_normal(32) * 1e-6).astype(np.float32)
            elif kind == 2:
                x = np.zeros(32, np.float32)
                x[rng.integers(0, 32)] = rng.choice([-1.0, 1.0]) * rng.uniform(0.5, 50.0)
            elif kind == 3:
                x = np.where(rng.integers(0, 2, 32) == 1, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
            elif kind == 4:
                x = (rng.standard_normal(32) * 1e4).astype(np.float32)
            else:
                x = rng.standard_normal(32).astype(np.float32)
            rows[t, g0:g0 + 32] = x
    if dtype == "bf16":
        rows = W.round_to_bf16(rows)
    assert np.all(np.isfinite(rows))
    return rows


# bf16 at 48 Queries runs the decode kernel, at 96 the prefill kernel
@pytest.mark.parametrize("name,n_q", [("tiny", 64), ("video_chunk", 48), ("video_chunk", 96)])
def test_quantize_degenerate_groups(name, n_q):
    """Quantize-append and attention over Keys and Values made of degenerate
    groups: the records equal the oracle's bit for bit and the outputs stay
    within 1e-3 of its rows."""
    n = 448
    w = small(W.workload(name), heads=1, n_kv=n, n_q=n_q)
    rng = np.random.default_rng(11)
    g = W.HeadGen(w, 0)
    C = W.round_to_bf16(g.keys(0, w.n_centroids)) if w.dtype == "bf16" else g.keys(0, w.n_centroids)
    S = O.sensitivity(g.hist_queries(), w.group)
    U = O.subspace(g.hist_queries(), w.rank)
    cals = [(C, S, U)]
    keys = [_degenerate_rows(rng, n, w.head_dim, w.dtype, C)]
    vals = [_degenerate_rows(rng, n, w.head_dim, w.dtype, C)]
    cache = _cache(w)
    import_calibration(cache, cals, w.dtype)
    cache.quantize_append(to_dev(keys, w.dtype), to_dev(vals, w.dtype))
    dec = cache.decode_export(cache.export().cpu().numpy(), n)
    rec = O.quantize_tokens(keys[0], vals[0], C, S, U, w.group)
    compare_records(dec, 0, rec)
    q = [g.current_queries()[:w.n_q]]
    out = cache.attend(to_dev(q, w.dtype)).cpu().numpy()
    ref = O.attend(q[0], _oracle_heads(w, keys, vals, cals)[0], None, None, mask="none")
    assert np.all(np.isfinite(out[0]))
    # the spread of logits is in the tens of thousands: some rows put all
    # their weight on a token whose Values are zero, so the reference row is
    # exactly 0 and the relative measure is undefined; those rows must be
    # (near) zero on the GPU too
    zero = np.abs(ref).max(axis=1) == 0
    e = row_rel_err(out[0][~zero], ref[~zero])
    log(f"  {name}: degenerate groups: records equal the oracle's, worst row error {e.max():.3e}, "
        f"{int(zero.sum())} all-zero rows")
    assert e.max() <= ROW_TOL
    assert np.abs(out[0][zero]).max(initial=0.0) <= 1e-6


def _oracle_heads(w, keys, vals, cals):
    hcs = []
    for h in range(w.heads):
        hc = O.HeadCache(w.group, w.dtype)
        hc.add_epoch(*cals[h])
        hc.append(keys[h], vals[h])
        hcs.append(hc)
    return hcs


# 49 Queries: the first count past the decode kernel's 48 (prefill path);
# 257: one live Query in the second 256-Query workgroup; 1000 Keys: a ragged
# last tile.
@pytest.mark.parametrize("name,heads,n_kv,n_q,mask", [
    ("tiny", 1, 1024, 16, "none"),
    ("video_chunk", 12, 7040, 880, "full"),
    ("video_chunk", 2, 1000, 200, "none"),
    ("video_chunk", 2, 1000, 49, "none"),
    ("video_chunk", 2, 3001, 257, "none"),
])
def test_attend_matches_oracle(name, heads, n_kv, n_q, mask):
    w = small(W.workload(name), heads=heads, n_kv=n_kv, n_q=n_q, n_self=n_q if mask != "none" else 0)
    log(f"[attend parity] {name} H={heads} n_kv={n_kv} n_q={n_q} mask={mask}")
    gens, keys, vals, cals = _setup(w, n_kv, min(n_kv, 880), 2)
    cache = _cache(w)
    import_calibration(cache, cals, w.dtype)
    cache.quantize_append(to_dev(keys, w.dtype), to_dev(vals, w.dtype))
    q = [g.current_queries()[:n_q] for g in gens]
    ks = vs = None
    if mask != "none":
        ks = [g.keys(n_kv, n_kv + n_q) for g in gens]
        vs = [g.values(n_kv, n_kv + n_q) for g in gens]
        out = cache.attend(to_dev(q, w.dtype), to_dev(ks, w.dtype), to_dev(vs, w.dtype), mask=mask)
    else:
        out = cache.attend(to_dev(q, w.dtype))
    out = out.cpu().numpy()
    hcs = _oracle_heads(w, keys, vals, cals)
    worst = 0.0
    for h in range(heads):
        ref = O.attend(q[h], hcs[h], None if ks is None else ks[h], None if vs is None else vs[h], mask=mask)
        e = row_rel_err(out[h], ref)
        worst = max(worst, float(e.max()))
        assert e.max() <= ROW_TOL, f"head {h}: row error {e.max():.3e}"
    log(f"  worst row error {worst:.3e}")


@pytest.mark.parametrize("name,heads,n_kv,n_q", [("tiny", 1, 1024, 16), ("video_chunk", 2, 7040, 150)])
def test_logits_match_oracle(name, heads, n_kv, n_q):
    w = small(W.workload(name), heads=heads, n_kv=n_kv, n_q=n_q)
    log(f"[logits parity] {name}")
    gens, keys, vals, cals = _setup(w, n_kv, min(n_kv, 880), 2)
    cache = _cache(w)
    import_calibration(cache, cals, w.dtype)
    cache.quantize_append(to_dev(keys, w.dtype), to_dev(vals, w.dtype))
    q = [g.current_queries()[:n_q] for g in gens]
    qd = to_dev(q, w.dtype)
    hcs = _oracle_heads(w, keys, vals, cals)
    scale = 1.0 / np.sqrt(w.head_dim)
    for h in range(heads):
        got = cache.attend_logits(qd, h).cpu().numpy()
        ref = O.cache_logits(q[h], hcs[h], scale)
        e = row_rel_err(got, ref)
        log(f"  head {h}: worst logit row error {e.max():.3e}")
        assert e.max() <= ROW_TOL


def test_causal_self_segment_and_ragged_tiles():
    """Token-causal self segment; cache and chunk lengths not multiples of 64."""
    w = small(W.workload("video_chunk"), heads=2, n_kv=333, n_q=77, n_self=77)
    log("[causal self] H=2 n_kv=333 n_q=77")
    gens, keys, vals, cals = _setup(w, w.n_kv, 333, 2)
    cache = _cache(w)
    import_calibration(cache, cals, w.dtype)
    cache.quantize_append(to_dev(keys, w.dtype), to_dev(vals, w.dtype))
    q = [g.current_queries()[:77] for g in gens]
    ks = [g.keys(333, 410) for g in gens]
    vs = [g.values(333, 410) for g in gens]
    out = cache.attend(to_dev(q, w.dtype), to_dev(ks, w.dtype), to_dev(vs, w.dtype), mask="causal").cpu().numpy()
    hcs = _oracle_heads(w, keys, vals, cals)
    for h in range(2):
        ref = O.attend(q[h], hcs[h], ks[h], vs[h], mask="causal")
        assert row_rel_err(out[h], ref).max() <= ROW_TOL


def test_multi_epoch_cache():
    """Three epochs with different calibrations and ragged epoch lengths;
    tokens keep their epoch's centroids and subspace."""
    w = small(W.workload("video_chunk"), heads=2, n_q=96)
    lens = [700, 1300, 419]
    log(f"[multi-epoch] lens={lens}")
    gens = [W.HeadGen(w, h) for h in range(2)]
    cache = _cache(w, capacity=sum(lens), max_epochs=3, max_q=96)
    hcs = [O.HeadCache(w.group, w.dtype) for _ in range(2)]
    t = 0
    allk, allv = [[], []], [[], []]
    for e, n in enumerate(lens):
        keys = [g.keys(t, t + n) for g in gens]
        vals = [g.values(t, t + n) for g in gens]
        cals = [oracle_calibration(w, g, k[:300], g.hist_queries(e), 1) for g, k in zip(gens, keys)]
        import_calibration(cache, cals, w.dtype)
        cache.quantize_append(to_dev(keys, w.dtype), to_dev(vals, w.dtype))
        for h in range(2):
            hcs[h].add_epoch(*cals[h])
            hcs[h].append(keys[h], vals[h])
        t += n
    assert cache.epochs() == 3 and cache.length() == sum(lens)
    dec = cache.decode_export(cache.export().cpu().numpy(), sum(lens))
    for h in range(2):
        off = 0
        for (start, rec) in hcs[h].records:
            compare_records(dec, h, rec, start)
        assert np.array_equal(dec["epoch"][h], hcs[h].field("epoch"))
    q = [g.current_queries()[:96] for g in gens]
    out = cache.attend(to_dev(q, w.dtype)).cpu().numpy()
    for h in range(2):
        ref = O.attend(q[h], hcs[h])
        assert row_rel_err(out[h], ref).max() <= ROW_TOL


def test_append_in_pieces_and_truncate():
    w = small(W.workload("video_chunk"), heads=3, n_kv=1000)
    log("[append pieces / truncate]")
    gens, keys, vals, cals = _setup(w, 1000, 500, 1)
    a = _cache(w)
    import_calibration(a, cals, w.dtype)
    a.quantize_append(to_dev(keys, w.dtype), to_dev(vals, w.dtype))
    b = _cache(w)
    import_calibration(b, cals, w.dtype)
    for s in (0, 130, 131, 600):
        e = {0: 130, 130: 131, 131: 600, 600: 1000}[s]
        b.quantize_append(to_dev([k[s:e] for k in keys], w.dtype), to_dev([v[s:e] for v in vals], w.dtype))
    ea, eb = a.export().cpu().numpy(), b.export().cpu().numpy()
    assert np.array_equal(ea, eb)
    # rewind and append again: identical bits
    b.truncate(131)
    b.quantize_append(to_dev([k[131:] for k in keys], w.dtype), to_dev([v[131:] for v in vals], w.dtype))
    assert np.array_equal(b.export().cpu().numpy(), ea)


def test_determinism():
    w = small(W.workload("video_chunk"), heads=4, n_kv=2000, n_q=300, n_self=300)
    gens, keys, vals, cals = _setup(w, 2000, 500, 1)
    outs = []
    for _ in range(2):
        c = _cache(w)
        import_calibration(c, cals, w.dtype)
        c.quantize_append(to_dev(keys, w.dtype), to_dev(vals, w.dtype))
        q = [g.current_queries()[:300] for g in gens]
        ks = [g.keys(2000, 2300) for g in gens]
        vs = [g.values(2000, 2300) for g in gens]
        o = c.attend(to_dev(q, w.dtype), to_dev(ks, w.dtype), to_dev(vs, w.dtype), mask="full")
        outs.append((c.export().cpu().numpy(), o.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))


# wm_layer at 9000 Keys (256 centroids, at least 32 Keys per centroid) takes
# the pruned assignment after the first iteration; the others run the full
# pass (the pruned pass needs 128 or more centroids).
@pytest.mark.parametrize("name,heads,n_keys,iters,seed", [("tiny", 1, 1024, 10, 0), ("video_chunk", 4, 1760, 4, 0),
                                                          ("video_chunk", 2, 4000, 4, 0), ("wm_layer", 2, 1560, 4, 0),
                                                          ("wm_layer", 2, 9000, 4, 0), ("wm_layer", 1, 9000, 3, 1),
                                                          ("video_chunk", 2, 1760, 4, 2)])
def test_build_calibration(name, heads, n_keys, iters, seed):
    """GPU-built calibration: S_G bit-exact (exact float64 sums of bf16/fp32
    squares), U_r spans the oracle's subspace (projector within 1e-4), and the
    GPU k-means reaches the oracle's mean QSAC objective within 1% (bf16
    Keys: the oracle's centroids bit for bit)."""
    w = small(W.workload(name), heads=heads)
    log(f"[build] {name} H={heads} n_keys={n_keys} iters={iters} seed={seed}")
    gens = [W.HeadGen(w, h, seed) for h in range(heads)]
    qh = [g.hist_queries() for g in gens]
    keys = [g.keys(0, n_keys) for g in gens]
    cache = _cache(w, max_build=n_keys)
    cache.build_subspace(to_dev(qh, w.dtype))
    cache.build_centroids(to_dev(keys, w.dtype), iters)
    C, S, U = (t.cpu() for t in cache.export_calibration(0))
    C = C.float().numpy()
    S = S.numpy()
    U = U.numpy()
    for h in range(heads):
        So = O.sensitivity(qh[h], w.group)
        Uo = O.subspace(qh[h], w.rank)
        if w.dtype == "bf16":
            assert np.array_equal(S[h], So), (S[h], So)  # exact float64 sums of bf16 squares
        else:
            assert np.all(np.abs(S[h] - So) <= np.spacing(So)), (S[h], So)
        P1 = U[h].astype(np.float64) @ U[h].astype(np.float64).T
        P2 = Uo.astype(np.float64) @ Uo.astype(np.float64).T
        perr = np.linalg.norm(P1 - P2) / np.linalg.norm(P2)
        log(f"  head {h}: projector error {perr:.2e}")
        assert perr < 1e-4
        Co = O.build_centroids(keys[h], So, w.n_centroids, w.group, iters, w.dtype)
        jg = O.mean_objective(keys[h], C[h], So, w.group)
        jo = O.mean_objective(keys[h], Co, So, w.group)
        log(f"  head {h}: mean J gpu {jg:.6g} oracle {jo:.6g} bit-identical centroids {np.array_equal(C[h], Co)}")
        assert abs(jg - jo) <= 0.01 * jo
        if w.dtype == "bf16":
            # float64 sums of bf16 Keys are exact in any order, and the ids are
            # bit-exact: the centroids are the oracle's bits
            assert np.array_equal(C[h], Co)


# The work counter behind the k-means roofline: a full assignment pass makes
# heads x Keys x centroids x head_dim channel evaluations; the pruned pass
# counts what its waves computed, at least the previous centroid's cost of
# every Key and at most the full pass. Profiling must not change the result.
@pytest.mark.parametrize("name,heads,n_keys,iters", [("video_chunk", 2, 1760, 3), ("wm_layer", 2, 9000, 3)])
def test_assign_work_counter(name, heads, n_keys, iters):
    w = small(W.workload(name), heads=heads)
    log(f"[work] {name} H={heads} n_keys={n_keys} iters={iters}")
    gens = [W.HeadGen(w, h, 0) for h in range(heads)]
    qh = to_dev([g.hist_queries() for g in gens], w.dtype)
    keys = to_dev([g.keys(0, n_keys) for g in gens], w.dtype)
    Cs, works = [], []
    for prof in (False, True):
        cache = _cache(w, max_build=n_keys)
        cache.profile_enable(prof)
        cache.build_subspace(qh)
        cache.build_centroids(keys, iters)
        Cs.append(cache.export_calibration(0)[0].cpu())
        works.append(cache.profile_work("assign"))
        cache.profile_enable(False)
    assert torch.equal(Cs[0].view(torch.int16) if Cs[0].dtype == torch.bfloat16 else Cs[0],
                       Cs[1].view(torch.int16) if Cs[1].dtype == torch.bfloat16 else Cs[1])
    assert works[0] == 0.0
    full = float(heads * n_keys * w.n_centroids * w.head_dim)
    log(f"  evaluations {works[1]:.6g} = {works[1] / full:.3f} full passes")
    if w.n_centroids < 128:
        assert works[1] == iters * full
    else:
        floor = full + (iters - 1) * float(heads * n_keys * w.head_dim)
        assert floor <= works[1] <= iters * full
        assert works[1] < 0.9 * iters * full  # the bound skips work on this data


# Builds at the edges of the k-means kernels: fewer Keys than centroids
# (duplicate seeds that never win a tie), a single Key, and odd Key counts
# whose per-head id rows start off a 16-byte boundary (the update kernel reads
# the ids as aligned 16-byte blocks and masks the bytes outside the head),
# on both update shapes (2 waves up to 4,096 Keys, 8 beyond).
@pytest.mark.parametrize("name,heads,n_keys,iters", [("tiny", 1, 1, 3), ("tiny", 1, 5, 3),
                                                     ("video_chunk", 3, 37, 3), ("video_chunk", 2, 70, 2),
                                                     ("video_chunk", 3, 4097, 2)])
def test_build_small_and_ragged(name, heads, n_keys, iters):
    w = small(W.workload(name), heads=heads)
    log(f"[build edge] {name} H={heads} n_keys={n_keys} iters={iters}")
    gens = [W.HeadGen(w, h) for h in range(heads)]
    qh = [g.hist_queries() for g in gens]
    keys = [g.keys(0, n_keys) for g in gens]
    cache = _cache(w, max_build=n_keys)
    cache.build_subspace(to_dev(qh, w.dtype))
    cache.build_centroids(to_dev(keys, w.dtype), iters)
    C = cache.export_calibration(0)[0].cpu().float().numpy()
    for h in range(heads):
        So = O.sensitivity(qh[h], w.group)
        Co = O.build_centroids(keys[h], So, w.n_centroids, w.group, iters, w.dtype)
        same = np.array_equal(C[h], Co)
        log(f"  head {h}: identical centroids {same}")
        if w.dtype == "bf16":
            assert same
        else:
            jg = O.mean_objective(keys[h], C[h], So, w.group)
            jo = O.mean_objective(keys[h], Co, So, w.group)
            assert abs(jg - jo) <= 0.01 * max(jo, 1e-30)


# The most epochs a cache holds (64), most of them shorter than one 64-token
# tile: the prefill kernel's tile ring and segment cursor step through
# segments of 1 to 100 tokens, the q.U and q.C tables span 64 epochs, and with
# a self segment the plan holds its most segments (65).
@pytest.mark.parametrize("n_q,mask", [(16, "none"), (96, "none"), (48, "full")])
def test_max_epochs_short_segments(n_q, mask):
    from video_world_model_amd import Cache
    w = small(W.workload("video_chunk"), heads=2, n_centroids=16, rank=8)
    rng = np.random.default_rng(64)
    lens = [int(x) for x in rng.integers(1, 101, size=64)]
    lens[5] = 64  # one epoch of exactly one tile
    total = sum(lens)
    log(f"[64 epochs] total {total} tokens, n_q={n_q}, mask={mask}")
    gens = [W.HeadGen(w, h, 3) for h in range(2)]
    keys = [g.keys(0, total + n_q) for g in gens]
    vals = [g.values(0, total + n_q) for g in gens]
    cache = Cache(2, w.head_dim, w.n_centroids, w.rank, total, dtype=torch.bfloat16, max_epochs=64,
                  max_query_tokens=max(n_q, 16), max_build_tokens=64)
    hcs = [O.HeadCache(w.group, w.dtype) for _ in range(2)]
    t = 0
    for e, n in enumerate(lens):
        cals = []
        for h in range(2):
            qh = gens[h].hist_queries(e % 8)
            S = O.sensitivity(qh, w.group)
            U = O.subspace(qh, w.rank)
            C = O.init_centroids(keys[h][t:t + max(n, w.n_centroids)], w.n_centroids)
            cals.append((C, S, U))
            hcs[h].add_epoch(C, S, U)
        import_calibration(cache, cals, w.dtype)
        cache.quantize_append(to_dev([k[t:t + n] for k in keys], w.dtype), to_dev([v[t:t + n] for v in vals], w.dtype))
        for h in range(2):
            hcs[h].append(keys[h][t:t + n], vals[h][t:t + n])
        t += n
    assert cache.epochs() == 64 and cache.length() == total
    dec = cache.decode_export(cache.export().cpu().numpy(), total)
    for h in range(2):
        for start, rec in hcs[h].records:
            compare_records(dec, h, rec, start)
        assert np.array_equal(dec["epoch"][h], hcs[h].field("epoch"))
    q = [g.current_queries()[:n_q] for g in gens]
    if mask == "none":
        out = cache.attend(to_dev(q, w.dtype)).cpu().numpy()
        ks = vs = [None, None]
    else:
        ks = [k[total:total + n_q] for k in keys]
        vs = [v[total:total + n_q] for v in vals]
        out = cache.attend(to_dev(q, w.dtype), to_dev(ks, w.dtype), to_dev(vs, w.dtype), mask=mask).cpu().numpy()
    worst = 0.0
    for h in range(2):
        ref = O.attend(q[h], hcs[h], ks[h], vs[h], mask=mask)
        e = row_rel_err(out[h], ref)
        worst = max(worst, float(e.max()))
        assert e.max() <= ROW_TOL
    log(f"  64 epochs: records bit-exact, worst row error {worst:.3e}")


# Empty inputs: an append of no tokens changes nothing, and a chunk attends to
# its own Keys alone while the cache holds no token yet (the plan's one
# segment is the self segment), with both self masks and on both kernels'
# dtypes.
@pytest.mark.parametrize("name,mask", [("video_chunk", "full"), ("video_chunk", "causal"), ("tiny", "causal")])
def test_empty_append_and_self_only(name, mask):
    n_q = 70
    w = small(W.workload(name), heads=2, n_q=n_q, n_self=n_q)
    log(f"[empty] {name} mask={mask}")
    g0 = [W.HeadGen(w, h) for h in range(2)]
    cals = [oracle_calibration(w, g, g.keys(0, 256), g.hist_queries(), 1) for g in g0]
    cache = _cache(w, capacity=512, max_q=n_q)
    import_calibration(cache, cals, w.dtype)
    empty = to_dev([g.keys(0, 1)[:0] for g in g0], w.dtype)
    cache.quantize_append(empty, empty)
    assert cache.length() == 0
    q = [g.current_queries()[:n_q] for g in g0]
    ks = [g.keys(300, 300 + n_q) for g in g0]
    vs = [g.values(300, 300 + n_q) for g in g0]
    out = cache.attend(to_dev(q, w.dtype), to_dev(ks, w.dtype), to_dev(vs, w.dtype), mask=mask).cpu().numpy()
    for h in range(2):
        hc = O.HeadCache(w.group, w.dtype)
        hc.add_epoch(*cals[h])
        ref = O.attend(q[h], hc, ks[h], vs[h], mask=mask)
        assert row_rel_err(out[h], ref).max() <= ROW_TOL
    # then tokens, an empty append between two real ones: identical bytes
    keys = [g.keys(0, 200) for g in g0]
    vals = [g.values(0, 200) for g in g0]
    cache.quantize_append(to_dev([k[:120] for k in keys], w.dtype), to_dev([v[:120] for v in vals], w.dtype))
    before = cache.export().cpu().numpy()
    cache.quantize_append(empty, empty)
    assert cache.length() == 120 and np.array_equal(cache.export().cpu().numpy(), before)
