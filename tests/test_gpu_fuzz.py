"""GPU parity over seeded random configurations of the whole path, against
the CPU oracle, through the C ABI.

Each case draws a configuration:

- **Shape.** Heads 1-3; head_dim 64 or 128; bf16 or float32 inputs.
- **Calibration.** 1-256 centroids; PSAC rank 0-16 (odd ranks
  included); centroid rule QSAC, nearest (QVG) or the post-rounding error.
  Each epoch's calibration is built by the oracle from that epoch's Keys
  and its own historical Queries.
- **Cache.** 1-3 epochs of ragged lengths, each appended in one to three
  pieces.
- **Query chunk.** 1-300 Queries, so the bf16 head_dim-128 caches meet
  both the decode-shaped and the prefill kernels. The chunk optionally
  carries a full or causal self segment, and the softmax scale is the
  default, a random positive or a random negative value.

Bars as in the other parity tests:

- centroid ids, codes and fp16 parameters bit-exact;
- PSAC coefficients within one fp16 ulp;
- outputs within 1e-3 of the row's largest magnitude.

QuantWM itself: roboind.com article, "Step 1" (centroid and INT2 residual)
and "Step 2" (compensation in the Query subspace); fugumt.com abstract
(strictly causal: tokens keep the calibration of their epoch)."""

import numpy as np
import pytest

import oracle.qwm_oracle as O
import workloads as W
from tests.gpu_helpers import ROW_TOL, compare_records, log, row_rel_err, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = 48
G = 32


def _round(x, dtype):
    x = np.asarray(x, np.float32)
    return W.round_to_bf16(x) if dtype == "bf16" else x


def _config(i):
    rng = np.random.default_rng(4242 + i)
    d = int(rng.choice([64, 128], p=[0.3, 0.7]))
    dtype = "bf16" if rng.random() < 0.75 else "f32"
    cfg = dict(
        d=d, dtype=dtype, heads=int(rng.integers(1, 4)),
        m=int(rng.choice([1, 3, 16, 64, 200, 256])),
        r=int(rng.choice([0, 2, 3, 4, 8, 13, 16])),
        objective=str(rng.choice(["qsac", "qsac", "nearest", "postq"])),
        lens=[int(x) for x in rng.integers(1, 600, size=int(rng.integers(1, 4)))],
        n_q=int(rng.choice([1, 5, 16, 17, 40, 64, 65, 100, 224, 300])),
        mask=str(rng.choice(["none", "none", "full", "causal"])),
        scale=[None, float(rng.uniform(0.02, 0.3)), -float(rng.uniform(0.02, 0.3))][int(rng.integers(0, 3))],
        seed=4242 + i,
    )
    if cfg["objective"] == "nearest" and rng.random() < 0.5:
        cfg["r"] = 0
    return cfg


def _keys(rng, n, d, centers, spread):
    lab = rng.integers(0, len(centers), size=n)
    x = centers[lab] + 0.5 * rng.standard_normal((n, d))
    return (x * spread).astype(np.float32)


@pytest.mark.parametrize("case", range(N_CASES))
def test_fuzz_configuration(case):
    from video_world_model_amd import Cache
    c = _config(case)
    d, dtype, H, m, r, obj = c["d"], c["dtype"], c["heads"], c["m"], c["r"], c["objective"]
    log(f"[fuzz {case}] {c}")
    rng = np.random.default_rng(c["seed"])
    n_tot = sum(c["lens"])
    n_self = c["n_q"] if c["mask"] != "none" else 0
    # per-head generators: mixture Keys with a few heavy channels, Values,
    # low-rank historical Queries and current Queries
    centers = [rng.standard_normal((8, d)) for _ in range(H)]
    spread = []
    for _ in range(H):
        s = np.exp(0.5 * rng.standard_normal(d))
        s[rng.choice(d, size=2, replace=False)] *= 10.0
        spread.append(s.astype(np.float32))
    keys = [_round(_keys(rng, n_tot + n_self, d, centers[h], spread[h]), dtype) for h in range(H)]
    vals = [_round(rng.standard_normal((n_tot + n_self, d)) * rng.uniform(0.2, 3.0), dtype) for h in range(H)]
    basis = [rng.standard_normal((d, 8)) for _ in range(H)]

    def hist(h):
        z = rng.standard_normal((96, 8)) @ basis[h].T + 0.1 * rng.standard_normal((96, d))
        return _round(2.0 * z, dtype)

    q = [_round(2.0 * (rng.standard_normal((c["n_q"], 8)) @ basis[h].T + 0.1 * rng.standard_normal((c["n_q"], d))),
                dtype) for h in range(H)]

    cache = Cache(H, d, m, r, n_tot, dtype=torch_dtype(dtype), max_epochs=len(c["lens"]),
                  max_query_tokens=max(c["n_q"], 16), max_build_tokens=64, objective=obj)
    hcs = [O.HeadCache(G, dtype, obj) for _ in range(H)]
    t = 0
    for e, n in enumerate(c["lens"]):
        cals = []
        for h in range(H):
            qh = hist(h)
            S = O.sensitivity(qh, G)
            U = O.subspace(qh, r)
            C = O.build_centroids(keys[h][t:t + min(n, 300)], S, m, G, 1, dtype, objective=obj)
            cals.append((C, S, U))
            hcs[h].add_epoch(C, S, U)
        Cd = to_dev([cc[0] for cc in cals], dtype)
        Sd = torch.from_numpy(np.stack([cc[1] for cc in cals])).cuda()
        Ud = torch.from_numpy(np.ascontiguousarray(np.stack([cc[2] for cc in cals]))).cuda()
        cache.import_calibration(Cd, Sd, Ud)
        # the epoch's tokens in one to three pieces
        cuts = sorted(set([0, n] + [int(x) for x in rng.integers(1, n, size=int(rng.integers(0, 3)))] if n > 1 else [0, n]))
        for a, b in zip(cuts[:-1], cuts[1:]):
            cache.quantize_append(to_dev([k[t + a:t + b] for k in keys], dtype),
                                  to_dev([v[t + a:t + b] for v in vals], dtype))
            for h in range(H):
                hcs[h].append(keys[h][t + a:t + b], vals[h][t + a:t + b])
        t += n
    assert cache.length() == n_tot and cache.epochs() == len(c["lens"])

    dec = cache.decode_export(cache.export().cpu().numpy(), n_tot)
    for h in range(H):
        for start, rec in hcs[h].records:
            compare_records(dec, h, rec, start)
        assert np.array_equal(dec["epoch"][h], hcs[h].field("epoch"))

    ks = vs = None
    if n_self:
        ks = [k[n_tot:] for k in keys]
        vs = [v[n_tot:] for v in vals]
        out = cache.attend(to_dev(q, dtype), to_dev(ks, dtype), to_dev(vs, dtype), mask=c["mask"], scale=c["scale"])
    else:
        out = cache.attend(to_dev(q, dtype), scale=c["scale"])
    out = out.cpu().numpy()
    worst = 0.0
    for h in range(H):
        ref = O.attend(q[h], hcs[h], None if ks is None else ks[h], None if vs is None else vs[h], mask=c["mask"],
                       scale=c["scale"])
        assert np.all(np.isfinite(out[h]))
        e = row_rel_err(out[h], ref)
        worst = max(worst, float(e.max()))
        assert e.max() <= ROW_TOL, f"head {h}: row error {e.max():.3e}"
    log(f"  records bit-exact, worst row error {worst:.3e}")
