"""C-ABI checks that need no GPU: the library loads, exports every function
include/qwm.h declares, and its host-side argument/state checks return the
documented status codes before anything would be enqueued."""

import ctypes
import os
import re

import pytest

import video_world_model_amd.qwm as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "qwm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qwm_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) == 23
    L = Q.lib()
    for n in names:
        assert hasattr(L, n), n


def _desc(**kw):
    base = dict(heads=2, head_dim=128, n_centroids=16, rank=8, capacity_tokens=1000, dtype=Q.QWM_BF16,
                max_epochs=2, max_query_tokens=64, max_build_tokens=512)
    base.update(kw)
    return Q.make_desc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), Q.QWM_ERR_UNSUPPORTED),
    (dict(head_dim=256), Q.QWM_ERR_UNSUPPORTED),
    (dict(group=16), Q.QWM_ERR_UNSUPPORTED),
    (dict(n_centroids=0), Q.QWM_ERR_UNSUPPORTED),
    (dict(n_centroids=257), Q.QWM_ERR_UNSUPPORTED),
    (dict(rank=-1), Q.QWM_ERR_UNSUPPORTED),
    (dict(rank=17), Q.QWM_ERR_UNSUPPORTED),
    (dict(objective=3), Q.QWM_ERR_INVALID_ARG),
    (dict(objective=-1), Q.QWM_ERR_INVALID_ARG),
    (dict(max_epochs=65), Q.QWM_ERR_UNSUPPORTED),
    (dict(heads=0), Q.QWM_ERR_INVALID_ARG),
    (dict(dtype=7), Q.QWM_ERR_INVALID_ARG),
    (dict(capacity_tokens=0), Q.QWM_ERR_INVALID_ARG),
    (dict(max_query_tokens=0), Q.QWM_ERR_INVALID_ARG),
])
def test_desc_validation(kw, status):
    d = _desc(**kw)
    n = ctypes.c_size_t(0)
    assert Q.lib().qwm_arena_bytes(ctypes.byref(d), ctypes.byref(n)) == status
    assert Q.last_error()


@pytest.mark.parametrize("kw", [dict(rank=0), dict(objective=1), dict(rank=0, objective=1), dict(rank=16),
                                dict(objective=2)])
def test_desc_modes_accepted(kw):
    """Rank 0 (PSAC off) and the nearest-centroid rule (QVG) are valid caches;
    rank 0 needs fewer arena bytes (no coefficients, no basis)."""
    d = _desc(**kw)
    n = ctypes.c_size_t(0)
    assert Q.lib().qwm_arena_bytes(ctypes.byref(d), ctypes.byref(n)) == Q.QWM_OK
    if kw.get("rank") == 0:
        assert n.value < Q.arena_bytes(_desc())


def test_arena_bytes_accounts_for_every_region():
    d = _desc()
    nbytes = Q.arena_bytes(d)
    H, D, cap, r, m = 2, 128, 1024, 8, 16  # capacity rounded to a 64-token tile
    per_token = 2 * (D // 4) + 2 * (D // 32) * 4 + 1 + 2 * r
    assert nbytes >= H * cap * per_token + 3 * H * m * D * 2
    assert nbytes % 256 == 0


def _device_may_be_visible() -> bool:
    """True where a HIP device could be found. The handles below sit on a fake
    arena address, so a call that passes every check would enqueue kernels
    against unmapped memory on such a host: those calls are made only where
    no device exists, where they must fail with QWM_ERR_HIP after their
    checks. (Counting devices does not initialize the runtime.)"""
    if os.path.exists("/dev/kfd"):
        return True
    import torch
    return torch.cuda.device_count() > 0


@pytest.mark.parametrize("kw", [dict(), dict(rank=0), dict(rank=16, n_centroids=256), dict(dtype=Q.QWM_F32, head_dim=64,
                                                                                      rank=4, n_centroids=16)])
@pytest.mark.parametrize("n_tokens,n_epochs", [(0, 0), (1, 1), (777, 2), (1000, 2)])
def test_storage_bytes_equals_the_oracle_accounting(kw, n_tokens, n_epochs):
    """The library's stored bytes (from its arena layout) give the oracle's
    compression ratio: packed bytes per token-head plus the per-epoch tables
    (roboind.com article, "Figure 4": centroids, quantization parameters and
    compensation data all count)."""
    import oracle.qwm_oracle as O
    d = _desc(**kw)
    rb, tb = Q.storage_bytes(d, n_tokens, n_epochs)
    H, D, m, r = d.heads, d.head_dim, d.n_centroids, d.rank
    esz = 2 if d.dtype == Q.QWM_BF16 else 4
    assert rb == H * n_tokens * O.bytes_per_token_head(D, 32, r)
    assert tb == n_epochs * H * O.table_bytes_per_head_epoch(D, 32, m, r, esz)
    if n_tokens and n_epochs:
        ratio = H * n_tokens * 4 * D / (rb + tb)
        assert ratio == pytest.approx(O.compression_ratio(n_tokens, D, 32, m, r, esz, n_epochs), rel=1e-12)
    L = Q.lib()
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.qwm_storage_bytes(ctypes.byref(d), d.capacity_tokens + 1, 0, ctypes.byref(a), ctypes.byref(b)) == \
        Q.QWM_ERR_INVALID_ARG
    assert L.qwm_storage_bytes(ctypes.byref(d), 0, d.max_epochs + 1, ctypes.byref(a), ctypes.byref(b)) == \
        Q.QWM_ERR_INVALID_ARG
    assert L.qwm_storage_bytes(ctypes.byref(d), 0, 0, None, ctypes.byref(b)) == Q.QWM_ERR_INVALID_ARG


def _handle(**kw):
    d = _desc(**kw)
    h = ctypes.c_void_p()
    st = Q.lib().qwm_create(ctypes.byref(d), ctypes.c_void_p(1 << 20), Q.arena_bytes(d), None, ctypes.byref(h))
    assert st == Q.QWM_OK, Q.last_error()
    return h


def test_create_checks_arena():
    d = _desc()
    h = ctypes.c_void_p()
    L = Q.lib()
    need = Q.arena_bytes(d)
    assert L.qwm_create(ctypes.byref(d), None, need, None, ctypes.byref(h)) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_create(ctypes.byref(d), ctypes.c_void_p(256 + 16), need, None, ctypes.byref(h)) == \
        Q.QWM_ERR_ARENA_TOO_SMALL
    assert L.qwm_create(ctypes.byref(d), ctypes.c_void_p(256), need - 1, None, ctypes.byref(h)) == \
        Q.QWM_ERR_ARENA_TOO_SMALL
    assert L.qwm_create(ctypes.byref(d), ctypes.c_void_p(256), need, None, None) == Q.QWM_ERR_INVALID_ARG


def test_call_order_and_argument_checks():
    """State, capacity and argument errors are reported before any launch."""
    L = Q.lib()
    h = _handle()
    P = ctypes.c_void_p(4096)
    out = ctypes.c_void_p(8192)
    assert L.qwm_quantize_append(h, P, P, 10) == Q.QWM_ERR_STATE
    assert L.qwm_attend(h, P, 4, None, None, 0, 0, ctypes.c_float(0.1), out) == Q.QWM_ERR_STATE
    assert L.qwm_build_centroids(h, P, 100, 3) == Q.QWM_ERR_STATE
    assert L.qwm_build_centroids(h, P, 513, 3) == Q.QWM_ERR_CAPACITY
    assert L.qwm_build_centroids(h, P, 0, 3) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_build_centroids(h, P, 10, -1) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_build_subspace(h, None, 10) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_build_subspace(h, ctypes.c_void_p(4096 + 2), 10) == Q.QWM_ERR_INVALID_ARG  # misaligned
    assert L.qwm_build_subspace(h, P, 0) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_quantize_append(h, P, None, 10) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_quantize_append(h, None, None, 0) == Q.QWM_ERR_STATE  # the state is checked first
    assert L.qwm_quantize_append(h, P, P, -1) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_attend(h, P, 65, None, None, 0, 0, ctypes.c_float(0.1), out) == Q.QWM_ERR_CAPACITY
    assert L.qwm_attend(h, P, 0, None, None, 0, 0, ctypes.c_float(0.1), out) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_attend(h, P, 4, None, None, 0, 5, ctypes.c_float(0.1), out) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_attend(h, P, 4, None, None, 3, 0, ctypes.c_float(0.1), out) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_attend(h, P, 4, P, P, 3, 2, ctypes.c_float(0.1), out) == Q.QWM_ERR_INVALID_ARG  # causal n_self != n_q
    assert L.qwm_attend(h, P, 4, P, None, 4, 1, ctypes.c_float(0.1), out) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_attend(h, P, 4, None, None, 0, 0, ctypes.c_float(float("nan")), out) == Q.QWM_ERR_INVALID_ARG
    # the allocation-free attention: the same checks, no max_query_tokens bound
    assert L.qwm_attend_noalloc(h, P, 4, None, None, 0, 0, ctypes.c_float(0.1), out) == Q.QWM_ERR_STATE
    assert L.qwm_attend_noalloc(h, P, 65, None, None, 0, 0, ctypes.c_float(0.1), out) == Q.QWM_ERR_STATE
    assert L.qwm_attend_noalloc(h, P, (1 << 24) + 1, None, None, 0, 0, ctypes.c_float(0.1), out) == \
        Q.QWM_ERR_CAPACITY
    assert L.qwm_attend_noalloc(h, P, 0, None, None, 0, 0, ctypes.c_float(0.1), out) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_attend_noalloc(h, P, 4, P, P, 3, 2, ctypes.c_float(0.1), out) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_attend_noalloc(h, P, 4, None, None, 0, 0, ctypes.c_float(0.1), None) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_truncate(h, 1) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_export_calibration(h, 0, P, None, None) == Q.QWM_ERR_INVALID_ARG
    n = ctypes.c_int64(-1)
    assert L.qwm_length(h, ctypes.byref(n)) == Q.QWM_OK and n.value == 0
    e = ctypes.c_int32(-1)
    assert L.qwm_epochs(h, ctypes.byref(e)) == Q.QWM_OK and e.value == 0
    nb = ctypes.c_size_t(0)
    assert L.qwm_export_bytes(h, 0, 1, ctypes.byref(nb)) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_export_bytes(h, 0, 0, ctypes.byref(nb)) == Q.QWM_OK and nb.value == 0
    assert L.qwm_profile_read(h, 99, ctypes.byref(ctypes.c_double()), ctypes.byref(ctypes.c_int64())) == \
        Q.QWM_ERR_INVALID_ARG
    ev = ctypes.c_double(-1.0)
    assert L.qwm_profile_work(h, 99, ctypes.byref(ev)) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_profile_work(h, 6, None) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_profile_work(h, 6, ctypes.byref(ev)) == Q.QWM_OK and ev.value == 0.0
    assert L.qwm_destroy(h) == Q.QWM_OK
    assert L.qwm_destroy(None) == Q.QWM_ERR_INVALID_ARG


def test_mode_state_rules_and_top1_checks():
    """build_centroids needs a staged subspace except for the nearest-centroid
    rule at rank 0 (QVG), which then gets past the state check and, on a host
    without a device, fails only for want of one. qwm_attend_top1 checks its
    arguments first. Every call that could pass all checks is skipped where
    a device may exist (the handles' arena address is fake)."""
    L = Q.lib()
    P = ctypes.c_void_p(4096)
    top = ctypes.c_void_p(8192)
    no_device = not _device_may_be_visible()
    for kw, status in ((dict(), Q.QWM_ERR_STATE), (dict(rank=0), Q.QWM_ERR_STATE),
                       (dict(objective=1), Q.QWM_ERR_STATE), (dict(rank=0, objective=1), None)):
        h = _handle(**kw)
        if status is not None:
            assert L.qwm_build_centroids(h, P, 100, 3) == status
        elif no_device:  # past the state check, stopped only by the missing device
            assert L.qwm_build_centroids(h, P, 100, 3) == Q.QWM_ERR_HIP, Q.last_error()
        assert L.qwm_destroy(h) == Q.QWM_OK
    h = _handle()
    assert L.qwm_attend_top1(h, P, 4, None, 0, top) == Q.QWM_ERR_STATE  # empty cache
    assert L.qwm_attend_top1(h, P, 4, None, 3, top) == Q.QWM_ERR_INVALID_ARG  # n_ref without k_ref
    assert L.qwm_attend_top1(h, P, 4, P, 0, top) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_attend_top1(h, P, 4, P, (1 << 22) + 1, top) == Q.QWM_ERR_CAPACITY
    assert L.qwm_attend_top1(h, P, 65, P, 10, top) == Q.QWM_ERR_CAPACITY
    assert L.qwm_attend_top1(h, P, 4, P, 10, None) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_attend_top1(h, P, 0, P, 10, top) == Q.QWM_ERR_INVALID_ARG
    # import without a basis is allowed only at rank 0
    assert L.qwm_import_calibration(h, P, P, None) == Q.QWM_ERR_INVALID_ARG
    assert L.qwm_destroy(h) == Q.QWM_OK
    h = _handle(rank=0, objective=1)
    if no_device:  # a valid import; only the missing device stops it
        assert L.qwm_import_calibration(h, P, None, None) == Q.QWM_ERR_HIP, Q.last_error()
    assert L.qwm_destroy(h) == Q.QWM_OK


def test_one_hip_runtime_per_process():
    """Loading the library before anything imported torch must still leave one
    HIP runtime mapped in the process (torch's), not two."""
    import subprocess
    import sys
    code = ("import video_world_model_amd.qwm as Q; Q.lib(); import torch; "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, check=True).stdout
    libs = eval(out.strip().splitlines()[-1])
    assert len(libs) == 1, libs


def test_no_oracle_in_product_path():
    """The product package never imports the oracle."""
    pkg = os.path.join(ROOT, "video_world_model_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f
