"""Seeded synthetic inputs shaped like the QuantWM workloads.

This module only draws random numbers and rounds them to the storage dtype of
the inputs (bf16 or fp32). It holds none of the method's arithmetic: no
sensitivity, centroids, quantization, compensation or attention. Both the CPU
oracle (through the tests and the bench) and the GPU path consume the arrays it
returns, so the two sides always see identical inputs.

The pages run trained video world models (LingBot-World-v2, HY-World 1.5,
Matrix-Game-2, LongCat-Video, Causal-Forcing); their weights and activations
are not available, so the five workloads below stand in for them with the
shapes the pages' setting implies: frames of 880 or 1,560 latent tokens per
head, head_dim 64/128, a Key distribution with clustered structure and a few
heavy outlier channels, and Queries whose energy sits in a few principal
directions. The Query spectrum is tuned so that about 70% of the energy lies in
the first 8 principal directions, matching the one such figure the QuantWM
article gives for a LingBot-World-v2 layer (roboind.com article, "Step 2").

Every array is generated per (workload, array kind, head, block) from its own
``numpy.random.SeedSequence``, so any head, frame or token range can be
produced on its own and always gives the same values.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "round_to_bf16",
    "bf16_bits",
    "HeadGen",
    "QUERY_ALPHA",
]

# Query amplitude: chosen so that attention logits q.k/sqrt(d) have a standard
# deviation of roughly 2 on these Key distributions (a peaked but not one-hot
# softmax).
QUERY_ALPHA = 3.0
# Per-direction energy decay of the Query signal and the isotropic noise level.
QUERY_DECAY = 0.7
QUERY_NOISE = 0.1
# Within-component standard deviation of the Key mixture.
KEY_COMPONENT_STD = 0.5


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload (all counts are per head; B=1 is folded into heads)."""

    name: str
    index: int
    heads: int
    head_dim: int
    group: int
    n_centroids: int
    rank: int
    dtype: str  # "f32" or "bf16": the dtype of K, V, Q and the centroid table
    n_kv: int  # tokens in the cache when the Query chunk attends
    n_q: int  # Queries in the attending chunk
    n_hist: int  # historical Queries per calibration
    n_self: int  # tokens of the chunk's own bf16 K/V segment (0 = none)
    self_mask: str  # "none", "full" or "causal"
    frame_tokens: int  # latent tokens per frame
    key_components: int
    channel_lognormal_sigma: float  # 0 = no per-channel log-normal scaling
    outlier_channels: int
    outlier_scale: float
    query_rank: int
    epoch_tokens: Optional[int]  # calibration refresh period in tokens (None = one epoch)
    drift_std: float  # per-frame drift of the mixture means
    n_append: int  # tokens quantize-appended by one streaming step (0 = cache built whole)
    kmeans_iters: int = 10

    @property
    def n_groups(self) -> int:
        return self.head_dim // self.group

    @property
    def n_epochs(self) -> int:
        if self.epoch_tokens is None:
            return 1
        return -(-self.n_kv // self.epoch_tokens)

    def epoch_start(self, e: int) -> int:
        return 0 if self.epoch_tokens is None else e * self.epoch_tokens

    def epoch_end(self, e: int) -> int:
        if self.epoch_tokens is None:
            return self.n_kv
        return min(self.n_kv, (e + 1) * self.epoch_tokens)

    def centroid_keys_range(self, e: int):
        """Token range whose Keys build epoch ``e``'s centroids.

        A one-epoch cache builds them from all of its Keys. With periodic
        refresh, only the frame inserted at the refresh is still available in
        full precision (older Keys were already quantized), so epoch ``e``
        clusters the first frame of the epoch.
        """
        if self.epoch_tokens is None:
            return 0, self.n_kv
        s = self.epoch_start(e)
        return s, min(self.n_kv, s + self.frame_tokens)


WORKLOADS: Dict[str, Workload] = {}


def _add(w: Workload) -> None:
    WORKLOADS[w.name] = w


# Tiny CPU-scale case: 1 head, d=64, fp32, 1,024 cached tokens.
_add(Workload(
    name="tiny", index=0, heads=1, head_dim=64, group=32, n_centroids=16, rank=4,
    dtype="f32", n_kv=1024, n_q=16, n_hist=64, n_self=0, self_mask="none",
    frame_tokens=1024, key_components=16, channel_lognormal_sigma=1.0,
    outlier_channels=0, outlier_scale=1.0, query_rank=8, epoch_tokens=None,
    drift_std=0.0, n_append=0))
# Small video chunk: 12 heads, 8 frames x 880 tokens cached, one frame of
# Queries attending to the cache plus its own (not yet cached) bf16 K/V.
_add(Workload(
    name="video_chunk", index=1, heads=12, head_dim=128, group=32, n_centroids=64, rank=8,
    dtype="bf16", n_kv=7040, n_q=880, n_hist=880, n_self=880, self_mask="full",
    frame_tokens=880, key_components=32, channel_lognormal_sigma=0.0,
    outlier_channels=4, outlier_scale=20.0, query_rank=16, epoch_tokens=None,
    drift_std=0.0, n_append=0))
# World-model layer: 40 heads, 21 frames x 1,560 tokens, 3-frame Query chunk.
_add(Workload(
    name="wm_layer", index=2, heads=40, head_dim=128, group=32, n_centroids=256, rank=16,
    dtype="bf16", n_kv=32760, n_q=4680, n_hist=4680, n_self=0, self_mask="none",
    frame_tokens=1560, key_components=32, channel_lognormal_sigma=0.0,
    outlier_channels=4, outlier_scale=20.0, query_rank=16, epoch_tokens=None,
    drift_std=0.0, n_append=0))
# Streaming insert: a 100,000-token cache, one 1,560-token frame appended per
# step, calibration refreshed every 8 frames from the last 8 frames' Queries.
_add(Workload(
    name="streaming", index=3, heads=40, head_dim=128, group=32, n_centroids=256, rank=16,
    dtype="bf16", n_kv=101560, n_q=1560, n_hist=12480, n_self=0, self_mask="none",
    frame_tokens=1560, key_components=32, channel_lognormal_sigma=0.0,
    outlier_channels=4, outlier_scale=20.0, query_rank=16, epoch_tokens=12480,
    drift_std=0.0, n_append=1560))
# Long horizon: 131,072 cached tokens with slow per-frame mean drift, a
# quarter-frame (390) Query chunk.
_add(Workload(
    name="long_horizon", index=4, heads=40, head_dim=128, group=32, n_centroids=256, rank=16,
    dtype="bf16", n_kv=131072, n_q=390, n_hist=4680, n_self=0, self_mask="none",
    frame_tokens=1560, key_components=32, channel_lognormal_sigma=0.0,
    outlier_channels=4, outlier_scale=20.0, query_rank=16, epoch_tokens=12480,
    drift_std=0.01, n_append=0))


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        for w in WORKLOADS.values():
            if w.index == name_or_index:
                return w
        raise KeyError(name_or_index)
    return WORKLOADS[name_or_index]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The bfloat16 bit patterns of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bf16-exact")
    return (u >> 16).astype(np.uint16)


# Array kinds (part of each seed).
_K_PARAMS, _K_KEYS, _K_VALUES, _K_QUERIES = 1, 2, 3, 4
# Query streams.
Q_CURRENT = 0  # the attending chunk
Q_HIST = 1  # historical Queries (calibration); epoch e uses stream Q_HIST + e


class HeadGen:
    """Generator for one head of one workload."""

    def __init__(self, w: Workload, head: int, seed: int = 0):
        self.w = w
        self.head = head
        self.base = 1000 + w.index + 7919 * seed
        rng = self._rng(_K_PARAMS, 0)
        d = w.head_dim
        self.mu = rng.standard_normal((w.key_components, d)).astype(np.float32)
        if w.drift_std > 0:
            self.delta = (w.drift_std * rng.standard_normal((w.key_components, d))).astype(np.float32)
        else:
            self.delta = None
        scale = np.ones(d, np.float32)
        if w.channel_lognormal_sigma > 0:
            scale = np.exp(w.channel_lognormal_sigma * rng.standard_normal(d)).astype(np.float32)
        if w.outlier_channels > 0:
            ch = rng.choice(d, size=w.outlier_channels, replace=False)
            scale[ch] *= np.float32(w.outlier_scale)
        self.channel_scale = scale
        basis, _ = np.linalg.qr(rng.standard_normal((d, w.query_rank)))
        self.q_basis = basis.astype(np.float64)
        self.q_sqrt_lambda = np.sqrt(QUERY_DECAY ** np.arange(w.query_rank))

    def _rng(self, kind: int, block: int) -> np.random.Generator:
        return np.random.default_rng(np.random.SeedSequence([self.base, kind, self.head, block]))

    def _store(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        return round_to_bf16(x) if self.w.dtype == "bf16" else x

    def _frame_keys(self, f: int) -> np.ndarray:
        w = self.w
        rng = self._rng(_K_KEYS, f)
        comp = rng.integers(0, w.key_components, size=w.frame_tokens)
        z = rng.standard_normal((w.frame_tokens, w.head_dim), dtype=np.float32)
        mu = self.mu[comp]
        if self.delta is not None:
            mu = mu + np.float32(f) * self.delta[comp]
        return (mu + np.float32(KEY_COMPONENT_STD) * z) * self.channel_scale

    def _frame_values(self, f: int) -> np.ndarray:
        rng = self._rng(_K_VALUES, f)
        return rng.standard_normal((self.w.frame_tokens, self.w.head_dim), dtype=np.float32)

    def _range(self, fn, t0: int, t1: int) -> np.ndarray:
        F = self.w.frame_tokens
        out = np.empty((t1 - t0, self.w.head_dim), np.float32)
        t = t0
        while t < t1:
            f = t // F
            a = t - f * F
            b = min(F, t1 - f * F)
            out[t - t0:t - t0 + (b - a)] = fn(f)[a:b]
            t += b - a
        return self._store(out)

    def keys(self, t0: int, t1: int) -> np.ndarray:
        """Keys of stream tokens [t0, t1) in the stored dtype (as float32 values)."""
        return self._range(self._frame_keys, t0, t1)

    def values(self, t0: int, t1: int) -> np.ndarray:
        return self._range(self._frame_values, t0, t1)

    def queries(self, stream: int, n: int) -> np.ndarray:
        """``n`` Queries of one stream: a rank-R signal with decaying energy plus noise."""
        w = self.w
        rng = self._rng(_K_QUERIES, stream)
        z = rng.standard_normal((n, w.query_rank)) * self.q_sqrt_lambda
        eps = rng.standard_normal((n, w.head_dim))
        q = QUERY_ALPHA * (z @ self.q_basis.T + QUERY_NOISE * eps)
        return self._store(q.astype(np.float32))

    # Convenience accessors for the standard roles of each workload.
    def cache_keys(self) -> np.ndarray:
        return self.keys(0, self.w.n_kv)

    def cache_values(self) -> np.ndarray:
        return self.values(0, self.w.n_kv)

    def self_keys(self) -> np.ndarray:
        return self.keys(self.w.n_kv, self.w.n_kv + self.w.n_self)

    def self_values(self) -> np.ndarray:
        return self.values(self.w.n_kv, self.w.n_kv + self.w.n_self)

    def current_queries(self) -> np.ndarray:
        return self.queries(Q_CURRENT, self.w.n_q)

    def hist_queries(self, epoch: int = 0) -> np.ndarray:
        return self.queries(Q_HIST + epoch, self.w.n_hist)
