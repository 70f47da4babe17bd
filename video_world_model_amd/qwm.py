"""ctypes binding of libqwm.so (the QuantWM 2-bit KV cache for MI355X).

Argument marshalling only: every computation runs in the library's HIP
kernels. PyTorch supplies device memory (the arena and the caller's tensors)
and the HIP stream. The C ABI is documented in include/qwm.h; the methods
below carry the same names.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqwm.so")

QWM_OK = 0
QWM_ERR_INVALID_ARG = -1
QWM_ERR_UNSUPPORTED = -2
QWM_ERR_CAPACITY = -3
QWM_ERR_STATE = -4
QWM_ERR_HIP = -5
QWM_ERR_ARENA_TOO_SMALL = -6
STATUS_NAMES = {
    0: "QWM_OK", -1: "QWM_ERR_INVALID_ARG", -2: "QWM_ERR_UNSUPPORTED", -3: "QWM_ERR_CAPACITY",
    -4: "QWM_ERR_STATE", -5: "QWM_ERR_HIP", -6: "QWM_ERR_ARENA_TOO_SMALL",
}
QWM_BF16, QWM_F32 = 0, 1
OBJECTIVES = {"qsac": 0, "nearest": 1, "postq": 2}
MASKS = {"none": 0, "full": 1, "causal": 2}
KERNELS = {"quantize": 0, "attend": 1, "merge": 2, "qu": 3, "gram": 4, "eigen": 5, "assign": 6,
           "update": 7, "other": 8}


class QwmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("n_centroids", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("max_epochs", ctypes.c_int32),
        ("capacity_tokens", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("objective", ctypes.c_int32),
        ("max_query_tokens", ctypes.c_int64),
        ("max_build_tokens", ctypes.c_int64),
    ]


_lib = None

_VP = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SIGS = {
    "qwm_arena_bytes": [ctypes.POINTER(Desc), ctypes.POINTER(ctypes.c_size_t)],
    "qwm_storage_bytes": [ctypes.POINTER(Desc), _I64, _I32, ctypes.POINTER(ctypes.c_size_t),
                          ctypes.POINTER(ctypes.c_size_t)],
    "qwm_create": [ctypes.POINTER(Desc), _VP, ctypes.c_size_t, _VP, ctypes.POINTER(_VP)],
    "qwm_destroy": [_VP],
    "qwm_build_subspace": [_VP, _VP, _I64],
    "qwm_build_centroids": [_VP, _VP, _I64, _I32],
    "qwm_quantize_append": [_VP, _VP, _VP, _I64],
    "qwm_attend": [_VP, _VP, _I64, _VP, _VP, _I64, _I32, ctypes.c_float, _VP],
    "qwm_attend_noalloc": [_VP, _VP, _I64, _VP, _VP, _I64, _I32, ctypes.c_float, _VP],
    "qwm_length": [_VP, ctypes.POINTER(_I64)],
    "qwm_epochs": [_VP, ctypes.POINTER(_I32)],
    "qwm_truncate": [_VP, _I64],
    "qwm_import_calibration": [_VP, _VP, _VP, _VP],
    "qwm_export_calibration": [_VP, _I32, _VP, _VP, _VP],
    "qwm_export_bytes": [_VP, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)],
    "qwm_export": [_VP, _I64, _I64, _VP],
    "qwm_attend_logits": [_VP, _VP, _I64, _I32, ctypes.c_float, _VP],
    "qwm_attend_top1": [_VP, _VP, _I64, _VP, _I64, _VP],
    "qwm_profile_enable": [_VP, _I32],
    "qwm_profile_read": [_VP, _I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I64)],
    "qwm_profile_work": [_VP, _I32, ctypes.POINTER(ctypes.c_double)],
}


def lib() -> ctypes.CDLL:
    """Load libqwm.so (built in-tree by video_world_model_amd.build)."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime under the same soname as the one
        # libqwm.so was linked against. Loading torch first makes libqwm.so
        # bind to that already-loaded runtime; loaded the other way round the
        # process would map two HIP runtimes, and the first GPU call crashes.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m video_world_model_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.qwm_last_error.restype = ctypes.c_char_p
        L.qwm_last_error.argtypes = []
        L.qwm_version.restype = ctypes.c_char_p
        L.qwm_version.argtypes = []
        _lib = L
    return _lib


def version() -> str:
    return lib().qwm_version().decode()


def loaded_source_hash() -> str:
    """Source hash stamped into the loaded library ("" when unstamped)."""
    v = version()
    return v.split("src:", 1)[1] if "src:" in v else ""


def check_build() -> str:
    """Raise unless the loaded library was built from the sources in this
    tree; returns the hash."""
    from video_world_model_amd.build import source_hash
    want, got = source_hash(), loaded_source_hash()
    if got != want:
        raise RuntimeError(f"{LIB_PATH} was built from other sources (library src:{got or 'none'}, tree src:{want}); "
                           "rebuild with `python -m video_world_model_amd.build`")
    return got


def last_error() -> str:
    return lib().qwm_last_error().decode()


def check(status: int) -> None:
    if status != QWM_OK:
        raise QwmError(status, last_error())


def make_desc(heads, head_dim, n_centroids, rank, capacity_tokens, dtype=QWM_BF16, max_epochs=1,
              max_query_tokens=1024, max_build_tokens=1024, group=32, objective=0) -> Desc:
    return Desc(heads, head_dim, group, n_centroids, rank, max_epochs, capacity_tokens, dtype, objective,
                max_query_tokens, max_build_tokens)


def arena_bytes(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    check(lib().qwm_arena_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def storage_bytes(desc: Desc, n_tokens: int, n_epochs: int):
    """(record bytes, calibration-table bytes) of the stored state at n_tokens
    tokens per head in n_epochs epochs (qwm_storage_bytes)."""
    rb, tb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    check(lib().qwm_storage_bytes(ctypes.byref(desc), n_tokens, n_epochs, ctypes.byref(rb), ctypes.byref(tb)))
    return int(rb.value), int(tb.value)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


class Cache:
    """A QuantWM cache whose arena is a torch uint8 tensor on ``device``.

    Tensors passed in must be contiguous, on the cache's device, in the
    cache dtype (``torch.bfloat16`` or ``torch.float32``), shaped
    [heads][n][head_dim]; outputs are float32. ``objective`` is the centroid
    rule ("qsac"; "nearest" for the QVG baseline; "postq" for the weighted
    error after INT2 quantization); rank 0 turns PSAC off.
    """

    def __init__(self, heads: int, head_dim: int, n_centroids: int, rank: int, capacity_tokens: int,
                 dtype=None, max_epochs: int = 1, max_query_tokens: int = 1024,
                 max_build_tokens: int = 1024, device=None, objective: str = "qsac"):
        import torch
        self.torch = torch
        if dtype is None:
            dtype = torch.bfloat16
        if dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("dtype must be torch.bfloat16 or torch.float32")
        self.dtype = dtype
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.heads, self.head_dim, self.n_centroids, self.rank = heads, head_dim, n_centroids, rank
        self.group = 32
        if objective not in OBJECTIVES:
            raise ValueError(f"objective must be one of {sorted(OBJECTIVES)}")
        self.objective = objective
        self.desc = make_desc(heads, head_dim, n_centroids, rank, capacity_tokens,
                              QWM_BF16 if dtype == torch.bfloat16 else QWM_F32, max_epochs,
                              max_query_tokens, max_build_tokens, objective=OBJECTIVES[objective])
        nbytes = arena_bytes(self.desc)
        with torch.cuda.device(self.device):
            self.arena = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            self.stream = torch.cuda.current_stream(self.device)
            h = _VP()
            check(lib().qwm_create(ctypes.byref(self.desc), _ptr(self.arena), nbytes,
                                   ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(h)))
        self._h = h

    # -- helpers --------------------------------------------------------------
    def _chk(self, t, name, n=None, dtype=None):
        torch = self.torch
        dtype = self.dtype if dtype is None else dtype
        if t.device != self.device:
            raise ValueError(f"{name} must be on {self.device}")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 3 or t.shape[0] != self.heads or t.shape[2] != self.head_dim:
            raise ValueError(f"{name} must be [heads={self.heads}][n][head_dim={self.head_dim}], got {tuple(t.shape)}")
        if n is not None and t.shape[1] != n:
            raise ValueError(f"{name} must have {n} tokens")
        return t

    def close(self):
        if getattr(self, "_h", None):
            check(lib().qwm_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- the path -------------------------------------------------------------
    def build_subspace(self, q_hist):
        self._chk(q_hist, "q_hist")
        check(lib().qwm_build_subspace(self._h, _ptr(q_hist), q_hist.shape[1]))

    def build_centroids(self, keys, iters: int = 10):
        self._chk(keys, "keys")
        check(lib().qwm_build_centroids(self._h, _ptr(keys), keys.shape[1], iters))

    def quantize_append(self, k, v):
        self._chk(k, "k")
        self._chk(v, "v", k.shape[1])
        check(lib().qwm_quantize_append(self._h, _ptr(k), _ptr(v), k.shape[1]))

    def attend(self, q, k_self=None, v_self=None, mask: str = "none", scale: Optional[float] = None, out=None):
        torch = self.torch
        self._chk(q, "q")
        nq = q.shape[1]
        ns = 0
        if mask != "none":
            self._chk(k_self, "k_self")
            ns = k_self.shape[1]
            self._chk(v_self, "v_self", ns)
        if scale is None:
            scale = 1.0 / float(np.sqrt(self.head_dim))
        if out is None:
            out = torch.empty((self.heads, nq, self.head_dim), dtype=torch.float32, device=self.device)
        else:
            self._chk(out, "out", nq, torch.float32)
        check(lib().qwm_attend(self._h, _ptr(q), nq, _ptr(k_self), _ptr(v_self), ns, MASKS[mask],
                               ctypes.c_float(scale), _ptr(out)))
        return out

    def attend_noalloc(self, q, out, k_self=None, v_self=None, mask: str = "none", scale: Optional[float] = None):
        """qwm_attend_noalloc: attend() with its scratch in the library's static
        device array; `out` [heads][n_q][head_dim] float32 is the caller's."""
        self._chk(q, "q")
        nq = q.shape[1]
        ns = 0
        if mask != "none":
            self._chk(k_self, "k_self")
            ns = k_self.shape[1]
            self._chk(v_self, "v_self", ns)
        if scale is None:
            scale = 1.0 / float(np.sqrt(self.head_dim))
        self._chk(out, "out", nq, self.torch.float32)
        check(lib().qwm_attend_noalloc(self._h, _ptr(q), nq, _ptr(k_self), _ptr(v_self), ns, MASKS[mask],
                                       ctypes.c_float(scale), _ptr(out)))
        return out

    def attend_logits(self, q, head: int, scale: Optional[float] = None):
        torch = self.torch
        self._chk(q, "q")
        if scale is None:
            scale = 1.0 / float(np.sqrt(self.head_dim))
        out = torch.empty((q.shape[1], self.length()), dtype=torch.float32, device=self.device)
        check(lib().qwm_attend_logits(self._h, _ptr(q), q.shape[1], head, ctypes.c_float(scale), _ptr(out)))
        return out

    def attend_top1(self, q, k_ref=None):
        """Per head and Query, the index of the token with the largest logit:
        over the cache (compensated logits) or, with k_ref, over those
        full-precision Keys. Returns int32 [heads][n_q]."""
        torch = self.torch
        self._chk(q, "q")
        nref = 0
        if k_ref is not None:
            self._chk(k_ref, "k_ref")
            nref = k_ref.shape[1]
        out = torch.empty((self.heads, q.shape[1]), dtype=torch.int32, device=self.device)
        check(lib().qwm_attend_top1(self._h, _ptr(q), q.shape[1], _ptr(k_ref), nref, _ptr(out)))
        return out

    def storage_bytes(self):
        """(record bytes, calibration-table bytes) the cache holds now."""
        return storage_bytes(self.desc, self.length(), self.epochs())

    def compression_ratio(self) -> float:
        """bf16 K/V bytes of the cached tokens over the bytes stored for them,
        centroids, parameters and PSAC data included."""
        rb, tb = self.storage_bytes()
        return self.heads * self.length() * 4 * self.head_dim / (rb + tb)

    def length(self) -> int:
        n = _I64(0)
        check(lib().qwm_length(self._h, ctypes.byref(n)))
        return int(n.value)

    def epochs(self) -> int:
        n = _I32(0)
        check(lib().qwm_epochs(self._h, ctypes.byref(n)))
        return int(n.value)

    def truncate(self, n_tokens: int):
        check(lib().qwm_truncate(self._h, n_tokens))

    # -- calibration transfer and inspection ----------------------------------
    def import_calibration(self, C, S, U):
        torch = self.torch
        if tuple(C.shape) != (self.heads, self.n_centroids, self.head_dim) or C.dtype != self.dtype:
            raise ValueError("C must be [heads][n_centroids][head_dim] in the cache dtype")
        if S is not None and (tuple(S.shape) != (self.heads, self.head_dim // 32) or S.dtype != torch.float32):
            raise ValueError("S must be [heads][head_dim/32] float32")
        if U is not None and (tuple(U.shape) != (self.heads, self.head_dim, self.rank) or U.dtype != torch.float32):
            raise ValueError("U must be [heads][head_dim][rank] float32")
        if self.rank == 0:
            U = None  # nothing to import
        for t in (C, S, U):
            if t is None:
                continue
            if t.device != self.device or not t.is_contiguous():
                raise ValueError("calibration tensors must be contiguous on the cache device")
        check(lib().qwm_import_calibration(self._h, _ptr(C), _ptr(S), _ptr(U)))

    def export_calibration(self, epoch: int = 0):
        torch = self.torch
        C = torch.empty((self.heads, self.n_centroids, self.head_dim), dtype=self.dtype, device=self.device)
        S = torch.empty((self.heads, self.head_dim // 32), dtype=torch.float32, device=self.device)
        U = torch.empty((self.heads, self.head_dim, self.rank), dtype=torch.float32, device=self.device)
        check(lib().qwm_export_calibration(self._h, epoch, _ptr(C), _ptr(S), _ptr(U)))
        return C, S, U

    def export(self, t0: int = 0, t1: Optional[int] = None):
        """Records of tokens [t0, t1) in the canonical layout (device uint8 tensor)."""
        torch = self.torch
        t1 = self.length() if t1 is None else t1
        n = ctypes.c_size_t(0)
        check(lib().qwm_export_bytes(self._h, t0, t1, ctypes.byref(n)))
        buf = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=self.device)
        check(lib().qwm_export(self._h, t0, t1, _ptr(buf)))
        return buf[: int(n.value)]

    def decode_export(self, buf: np.ndarray, n: int) -> dict:
        """Split a canonical export (host bytes) into per-field numpy arrays [heads][n]..."""
        D, nG, r, H = self.head_dim, self.head_dim // 32, self.rank, self.heads
        per = n * (D // 2 + 8 * nG + 1 + 2 * r + 2)
        out = {k: [] for k in ("kcode", "vcode", "kzp", "kscale", "vzp", "vscale", "ids", "coef", "epoch")}
        for h in range(H):
            b = buf[h * per:(h + 1) * per]
            o = 0

            def take(nbytes):
                nonlocal o
                x = b[o:o + nbytes]
                o += nbytes
                return x
            out["kcode"].append(take(n * D // 4).reshape(n, D // 4))
            out["vcode"].append(take(n * D // 4).reshape(n, D // 4))
            for f in ("kzp", "kscale", "vzp", "vscale"):
                out[f].append(take(2 * n * nG).copy().view(np.float16).reshape(n, nG))
            out["ids"].append(take(n))
            out["coef"].append(take(2 * n * r).copy().view(np.float16).reshape(n, r))
            out["epoch"].append(take(2 * n).copy().view(np.uint16))
        return {k: np.stack(v) for k, v in out.items()}

    # -- event timing -----------------------------------------------------------
    def profile_enable(self, on: bool = True):
        check(lib().qwm_profile_enable(self._h, 1 if on else 0))

    def profile_read(self, kernel: str):
        ms = ctypes.c_double(0)
        n = _I64(0)
        check(lib().qwm_profile_read(self._h, KERNELS[kernel], ctypes.byref(ms), ctypes.byref(n)))
        return float(ms.value), int(n.value)

    def profile_work(self, kernel: str) -> float:
        """Channel evaluations of the centroid rule made by `kernel` launches
        since profiling was enabled (qwm_profile_work)."""
        ev = ctypes.c_double(0)
        check(lib().qwm_profile_work(self._h, KERNELS[kernel], ctypes.byref(ev)))
        return float(ev.value)
