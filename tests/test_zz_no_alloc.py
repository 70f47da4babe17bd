"""qwm_attend_noalloc (the attention entry point for callers that cannot
allocate: its scratch is the library's static device array) against
qwm_attend on the same cache, through the C ABI: two calls in a row, the
second smaller, on the prefill path (with a self segment) and the decode
path; outputs within 1e-3 of the row maximum (the two may split the KV
sequence differently). A call whose tables exceed the array is refused
before anything is enqueued."""

import numpy as np
import pytest

import workloads as W
from tests.gpu_helpers import ROW_TOL, log, row_rel_err, small, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def test_noalloc_attend_matches_attend():
    from video_world_model_amd import Cache
    import video_world_model_amd.qwm as Q
    w = small(W.workload("video_chunk"), heads=4)
    H, n_kv = w.heads, 3001
    lens = (1700, n_kv - 1700)  # two epochs, ragged
    gens = [W.HeadGen(w, h) for h in range(H)]
    cache = Cache(H, w.head_dim, w.n_centroids, w.rank, n_kv, dtype=torch.bfloat16, max_epochs=2,
                  max_query_tokens=700, max_build_tokens=800)
    t = 0
    for e, n in enumerate(lens):
        cache.build_subspace(to_dev([g.queries(W.Q_HIST + e, 600) for g in gens], "bf16"))
        cache.build_centroids(to_dev([g.keys(t, t + 800) for g in gens], "bf16"), 3)
        cache.quantize_append(to_dev([g.keys(t, t + n) for g in gens], "bf16"),
                              to_dev([g.values(t, t + n) for g in gens], "bf16"))
        t += n
    cases = [  # (n_q, self tokens): prefill with a self segment, then a smaller decode-shaped call
        (700, 300),
        (40, 0),
    ]
    for nq, ns in cases:
        log(f"[noalloc] n_q={nq} n_self={ns}")
        q = to_dev([g.current_queries()[:nq] for g in gens], "bf16")
        if ns:
            ks = to_dev([g.keys(n_kv, n_kv + ns) for g in gens], "bf16")
            vs = to_dev([g.values(n_kv, n_kv + ns) for g in gens], "bf16")
            ref = cache.attend(q, ks, vs, mask="full")
            out = torch.full((H, nq, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
            cache.attend_noalloc(q, out, ks, vs, mask="full")
        else:
            ref = cache.attend(q)
            out = torch.full((H, nq, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
            cache.attend_noalloc(q, out)
        ref, got = ref.cpu().numpy(), out.cpu().numpy()
        assert np.all(np.isfinite(got))
        err = max(row_rel_err(got[h], ref[h]).max() for h in range(H))
        log(f"  worst row error against qwm_attend {err:.2e}, bit-identical {np.array_equal(got, ref)}")
        assert err <= ROW_TOL
    # beyond max_query_tokens: only the static array bounds this call
    nq = 880
    q = to_dev([g.current_queries()[:nq] for g in gens], "bf16")
    out = torch.empty((H, nq, w.head_dim), dtype=torch.float32, device="cuda")
    cache.attend_noalloc(q, out)
    assert np.all(np.isfinite(out.cpu().numpy()))
    # tables beyond the 64 MiB array: refused, nothing written
    nq = (64 << 20) // (H * 2 * 64) + 1
    q = torch.zeros((H, nq, w.head_dim), dtype=torch.bfloat16, device="cuda")
    out = torch.full((H, nq, w.head_dim), 7.0, dtype=torch.float32, device="cuda")  # full size all the same
    st = Q.lib().qwm_attend_noalloc(cache._h, q.data_ptr(), nq, None, None, 0, 0, 0.0883883, out.data_ptr())
    assert st == Q.QWM_ERR_CAPACITY, Q.last_error()
    assert "static scratch" in Q.last_error()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_noalloc_without_room_for_the_fp16_centroid_copy():
    """On the bf16 head_dim-128 prefill path qwm_attend reads an fp16 copy of
    the epochs' centroid tables made at the start of the call (in the cache's
    arena). The allocation-free call keeps that copy in its static array only
    where it fits; here it does not (16 heads x 64 epochs x 256 centroids x
    256 bytes = 64 MiB, next to the q . U table), so its kernels convert the
    bf16 rows of every tile instead. Both must agree, with and without a self
    segment, within the attention bar (the two may split the KV sequence
    differently)."""
    from video_world_model_amd import Cache
    import oracle.qwm_oracle as O
    H, D, m, r, E, G = 16, 128, 256, 16, 64, 32
    rng = np.random.default_rng(64)
    lens = [int(x) for x in rng.integers(17, 80, size=E)]  # ragged epochs: partial tiles
    n_kv = sum(lens)
    assert H * E * m * D * 2 == 64 << 20
    cache = Cache(H, D, m, r, n_kv, dtype=torch.bfloat16, max_epochs=E, max_query_tokens=96, max_build_tokens=64)
    basis = rng.standard_normal((H, D, 8))
    for e, n in enumerate(lens):
        C = W.round_to_bf16(rng.standard_normal((H, m, D)).astype(np.float32))
        S, U = [], []
        for h in range(H):
            qh = 2.0 * (rng.standard_normal((64, 8)) @ basis[h].T + 0.1 * rng.standard_normal((64, D)))
            qh = W.round_to_bf16(qh.astype(np.float32))
            S.append(O.sensitivity(qh, G))
            U.append(O.subspace(qh, r))
        cache.import_calibration(to_dev(list(C), "bf16"), torch.from_numpy(np.stack(S)).cuda(),
                                 torch.from_numpy(np.ascontiguousarray(np.stack(U))).cuda())
        k = W.round_to_bf16((C[:, rng.integers(0, m, n)] + 0.5 * rng.standard_normal((H, n, D))).astype(np.float32))
        v = W.round_to_bf16(rng.standard_normal((H, n, D)).astype(np.float32))
        cache.quantize_append(to_dev(list(k), "bf16"), to_dev(list(v), "bf16"))
    assert cache.epochs() == E and cache.length() == n_kv
    nq = 96  # past the decode kernel's 48: the prefill kernel
    q = W.round_to_bf16((2.0 * np.einsum("hqk,hdk->hqd", rng.standard_normal((H, nq, 8)), basis)).astype(np.float32))
    ks = W.round_to_bf16(rng.standard_normal((H, nq, D)).astype(np.float32))
    vs = W.round_to_bf16(rng.standard_normal((H, nq, D)).astype(np.float32))
    qd, kd, vd = to_dev(list(q), "bf16"), to_dev(list(ks), "bf16"), to_dev(list(vs), "bf16")
    for self_seg in (False, True):
        log(f"[noalloc, no room for the copy] H={H} epochs={E} n_kv={n_kv} n_q={nq} self={self_seg}")
        out = torch.full((H, nq, D), float("nan"), dtype=torch.float32, device="cuda")
        if self_seg:
            ref = cache.attend(qd, kd, vd, mask="causal")
            cache.attend_noalloc(qd, out, kd, vd, mask="causal")
        else:
            ref = cache.attend(qd)
            cache.attend_noalloc(qd, out)
        ref, got = ref.cpu().numpy(), out.cpu().numpy()
        assert np.all(np.isfinite(got))
        err = max(row_rel_err(got[h], ref[h]).max() for h in range(H))
        log(f"  worst row error against qwm_attend {err:.2e}")
        assert err <= ROW_TOL
