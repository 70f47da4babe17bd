"""Shared helpers of the GPU parity tests: move generator arrays to the
device, run the CPU oracle on the same arrays, and compare to the bar the
tests use (bit-exact integer/fp16 fields; 1 fp16 ulp for PSAC coefficients;
row-max-relative 1e-3 for logits and outputs)."""

from __future__ import annotations

import dataclasses
import sys

import numpy as np

import oracle.qwm_oracle as O
import workloads as W

ROW_TOL = 1e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def small(w: W.Workload, **kw) -> W.Workload:
    return dataclasses.replace(w, **kw)


def to_dev(arrs, dtype_name: str):
    import torch
    x = np.ascontiguousarray(np.stack(arrs).astype(np.float32))
    if dtype_name == "bf16":
        bits = W.bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(x).cuda()


def torch_dtype(dtype_name: str):
    import torch
    return torch.bfloat16 if dtype_name == "bf16" else torch.float32


def oracle_calibration(w: W.Workload, hg: W.HeadGen, keys: np.ndarray, q_hist: np.ndarray, iters: int):
    S = O.sensitivity(q_hist, w.group)
    U = O.subspace(q_hist, w.rank)
    C = O.build_centroids(keys, S, w.n_centroids, w.group, iters, w.dtype)
    return C, S, U


def import_calibration(cache, cals, dtype_name):
    import torch
    C = to_dev([c[0] for c in cals], dtype_name)
    S = torch.from_numpy(np.stack([c[1] for c in cals])).cuda()
    U = torch.from_numpy(np.ascontiguousarray(np.stack([c[2] for c in cals]))).cuda()
    cache.import_calibration(C, S, U)


def f16_ulp_close(a, b) -> np.ndarray:
    a = np.asarray(a, np.float16).astype(np.float64)
    b = np.asarray(b, np.float16).astype(np.float64)
    ulp = np.spacing(np.maximum(np.abs(a), np.abs(b)).astype(np.float16)).astype(np.float64)
    return np.abs(a - b) <= ulp


def compare_records(dec: dict, h: int, rec: dict, t0: int = 0):
    """Compare one head's exported records (from token t0) with oracle records."""
    n = len(rec["ids"])
    sl = slice(t0, t0 + n)
    assert np.array_equal(dec["ids"][h][sl], rec["ids"]), f"head {h}: centroid ids differ"
    assert np.array_equal(dec["kcode"][h][sl], O.pack2(rec["kcode"])), f"head {h}: K codes differ"
    assert np.array_equal(dec["vcode"][h][sl], O.pack2(rec["vcode"])), f"head {h}: V codes differ"
    for f in ("kzp", "kscale", "vzp", "vscale"):
        assert np.array_equal(dec[f][h][sl].view(np.uint16), rec[f].view(np.uint16)), f"head {h}: {f} differs"
    ok = f16_ulp_close(dec["coef"][h][sl], rec["coef"])
    assert ok.all(), f"head {h}: {np.count_nonzero(~ok)} PSAC coefficients beyond 1 fp16 ulp"
    return int(np.count_nonzero(dec["coef"][h][sl].view(np.uint16) != rec["coef"].view(np.uint16)))


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row max |got - ref| / max |ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.abs(got - ref).max(axis=-1) / np.abs(ref).max(axis=-1)
