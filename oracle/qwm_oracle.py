"""QuantWM CPU oracle: a plain, slow, obviously-correct statement of what the
2-bit KV-cache hot path computes.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check of
``__graft_entry__`` and the bench's CPU-baseline leg may import this module.
The product path (the HIP library and its Python binding) never imports,
links or calls it, and this module imports nothing from the product path.

Sources. The method is QuantWM (arXiv 2609.26425): the English abstract on
fugumt.com (QSAC picks Key centroids that suit INT2 by weighing both the
sensitivity of historical Queries and the range of the residual; PSAC puts the
Key error that remains back along the dominant Query subspace through a
low-rank projection), the Italian author abstract on ai.info (same two techniques,
training-free and strictly causal), and the roboind.com article, sections
"Step 1" (a Key is assigned a high-precision centroid and the Key-centroid
residual is quantized to 2 bits; the nearest centroid is not necessarily the
best one after quantization: the residual's dynamic range and which channels
matter to attention decide) and "Step 2" (historical Query energy concentrates
in a few principal directions; the Key error along them is kept in a low-rank
form and added back to the attention logits).

The pages give no equations. Where they leave a step open this module takes
the plainest reading consistent with them; every such reading is listed in
the readings table of the design notes and restated in the docstring of the
function that takes it.

Precision. Steps whose result is an integer or a stored fp16/bf16 value that
the GPU must reproduce bit for bit (QSAC objective and argmin, INT2 codes and
their fp16 parameters) run in float32 elementwise numpy operations in exactly
the order written: numpy float32 ufuncs round to nearest-even and never fuse.
Everything else runs in float64.

Per-head convention: ``d`` channels split into groups of ``g`` contiguous
channels (``nG = d // g``), ``m`` centroids, PSAC rank ``r``.
"""

from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64
ZERO32 = np.float32(0.0)
THREE32 = np.float32(3.0)


# ---------------------------------------------------------------------------
# Storage rounding helpers
# ---------------------------------------------------------------------------

def fp16_round_down(x: np.ndarray) -> np.ndarray:
    """Largest float16 value <= x (x float32).

    Nearest-even rounding followed by one step toward -inf when it landed
    above ``x``. Used for the INT2 zero-point so that the stored grid starts
    at or below the group minimum.
    """
    x = np.asarray(x, dtype=F32)
    h = x.astype(np.float16)
    above = h.astype(F32) > x
    if np.any(above):
        with np.errstate(over="ignore"):
            h = np.where(above, np.nextafter(h, np.float16(-np.inf)), h)
    return h


def fp16_round_up(x: np.ndarray) -> np.ndarray:
    """Smallest float16 value >= x (x float32). Used for the INT2 step size."""
    x = np.asarray(x, dtype=F32)
    h = x.astype(np.float16)
    below = h.astype(F32) < x
    if np.any(below):
        with np.errstate(over="ignore"):
            h = np.where(below, np.nextafter(h, np.float16(np.inf)), h)
    return h


def fp16_step_up(x: np.ndarray) -> np.ndarray:
    """Smallest float16 value s >= x (x float32, >= 0) such that 3 s is a
    float16 value too. Used for the INT2 step: every reconstruction offset
    code * s (code 0..3) is then exactly an fp16 value. Computed as
    fp16_round_up, then at most three steps of one fp16 ulp upward while 3 s
    (exact in float32) is not an fp16 value. Steps whose triple would exceed
    the fp16 range (group ranges of 65,472 or more) are outside the supported
    range."""
    s = fp16_round_up(x)
    with np.errstate(over="ignore", invalid="ignore"):
        for _ in range(3):
            t = s.astype(F32) * THREE32
            bad = t.astype(np.float16).astype(F32) != t
            if not np.any(bad):
                break
            s = np.where(bad, np.nextafter(s, np.float16(np.inf)), s)
    return s


def f64_to_fp16(x: np.ndarray) -> np.ndarray:
    """float64 -> float16, round to nearest, ties to even (one rounding)."""
    return np.asarray(x, dtype=F64).astype(np.float16)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 with a single round-to-nearest-even; returns float32.

    Rounds to float32 by truncation with a sticky low bit (round to odd), then
    to bfloat16 to nearest-even; float32 keeps 16 more significand bits than
    bfloat16, so the result equals one direct rounding of ``x``.
    """
    x = np.asarray(x, dtype=F64)
    f = x.astype(F32)
    # truncate toward zero
    over = np.abs(f.astype(F64)) > np.abs(x)
    f = np.where(over, np.nextafter(f, F32(0.0)), f).astype(F32)
    b = f.view(np.uint32).copy()
    inexact = f.astype(F64) != x
    b = np.where(inexact, b | np.uint32(1), b)
    b64 = b.astype(np.uint64)
    b64 = (b64 + 0x7FFF + ((b64 >> 16) & 1)) & 0xFFFF0000
    return b64.astype(np.uint32).view(F32)


def f64_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the cache's stored dtype ("f32" or "bf16"); returns float32."""
    if dtype == "f32":
        return np.asarray(x, dtype=F64).astype(F32)
    if dtype == "bf16":
        return f64_to_bf16(x)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# O1 -- historical-Query sensitivity
# ---------------------------------------------------------------------------

def sensitivity(q_hist: np.ndarray, g: int) -> np.ndarray:
    """Per-group Query sensitivity S_G (float32, shape [d // g]).

    The abstracts say QSAC weighs the sensitivity of historical Queries so as
    to cut the quantization error in the channels that matter most to
    attention; the
    article's "Step 1" says what matters is which channels' errors reach the
    attention score. The reading taken: a Key error e changes the logit q.e,
    whose mean square over historical Queries is, under a diagonal
    approximation, sum_j E[q_j^2] e_j^2. So channel j's sensitivity is the
    second moment s_j = mean_i q_ij^2, and a group's sensitivity is
    S_G = sum_{j in G} s_j, computed in float64 as
    (sum over i and j in G of q_ij^2) / M and stored as float32.
    """
    q = np.asarray(q_hist, dtype=F64)
    M, d = q.shape
    if M == 0:
        raise ValueError("no historical Queries")
    sq = (q * q).sum(axis=0)  # per channel
    group_sum = sq.reshape(d // g, g).sum(axis=1)
    return (group_sum / F64(M)).astype(F32)


# ---------------------------------------------------------------------------
# O6 -- PSAC principal subspace
# ---------------------------------------------------------------------------

def subspace(q_hist: np.ndarray, r: int) -> np.ndarray:
    """Top-r principal directions of the historical Queries, U_r [d][r] float32.

    "Step 2" of the article: the energy of historical Queries concentrates in
    a few principal directions (about 71% in the first 8 for one
    LingBot-World-v2 layer). Energy is the sum of squares, which is what the
    logits see, so the directions are the eigenvectors of the uncentered Gram
    matrix Q^T Q with the r largest eigenvalues, in descending order. Sign
    convention: each column's entry of largest magnitude is positive (lowest
    index on a tie).
    """
    q = np.asarray(q_hist, dtype=F64)
    gram = q.T @ q
    w, v = np.linalg.eigh(gram)
    order = np.argsort(-w, kind="stable")[:r]
    u = v[:, order].copy()
    for k in range(r):
        i = int(np.argmax(np.abs(u[:, k])))
        if u[i, k] < 0:
            u[:, k] = -u[:, k]
    return u.astype(F32)


# ---------------------------------------------------------------------------
# O2 -- QSAC objective and assignment
# ---------------------------------------------------------------------------

def qsac_objective(k: np.ndarray, C: np.ndarray, S: np.ndarray, g: int) -> np.ndarray:
    """QSAC cost J[n, c] of assigning Key n to centroid c (float32 [N][m]).

    "Step 1": in the baseline (QVG) each Key takes its nearest high-precision
    centroid and the Key-centroid residual is stored in 2 bits; QSAC instead
    picks the centroid by the residual's dynamic range and by how much each
    channel's error matters to attention. With per-group asymmetric INT2 the
    step of group G is R_G / 3 (R_G = max - min of the residual over the
    group), the rounding error variance is step^2 / 12, and weighting each
    channel by its sensitivity gives sum_G S_G R_G^2 / 108. The constant is
    dropped, so

        J = sum_G S_G * (max_{j in G} r_j - min_{j in G} r_j)^2,   r = k - c,

    evaluated in float32 in this order: r = k - c; per group mx, mn (signed
    zeros folded to +0); R = mx - mn; t = R * R; u = S_G * t; then
    J = ((u_0 + u_1) + u_2) + ... left to right.
    """
    k = np.asarray(k, dtype=F32)
    C = np.asarray(C, dtype=F32)
    S = np.asarray(S, dtype=F32)
    N, d = k.shape
    m = C.shape[0]
    nG = d // g
    J = None
    for G in range(nG):
        sl = slice(G * g, (G + 1) * g)
        r = k[:, None, sl] - C[None, :, sl]
        mx = r.max(axis=2) + ZERO32
        mn = r.min(axis=2) + ZERO32
        R = mx - mn
        t = R * R
        u = S[G] * t
        J = u if J is None else J + u
    assert J is not None and J.shape == (N, m)
    return J


def qsac_assign(k: np.ndarray, C: np.ndarray, S: np.ndarray, g: int, chunk: int = 2048) -> np.ndarray:
    """Centroid id per Key: argmin_c J, ties (equal float32 J) to the smallest id."""
    k = np.asarray(k, dtype=F32)
    out = np.empty(k.shape[0], np.int64)
    for a in range(0, k.shape[0], chunk):
        J = qsac_objective(k[a:a + chunk], C, S, g)
        out[a:a + chunk] = np.argmin(J, axis=1)  # first occurrence of the minimum
    return out


def nearest_assign(k: np.ndarray, C: np.ndarray) -> np.ndarray:
    """Euclidean-nearest centroid in float64 (used to pin the float32 rule below)."""
    k = np.asarray(k, dtype=F64)
    C = np.asarray(C, dtype=F64)
    d2 = ((k[:, None, :] - C[None, :, :]) ** 2).sum(axis=2)
    return np.argmin(d2, axis=1)


def nearest_objective(k: np.ndarray, C: np.ndarray, g: int) -> np.ndarray:
    """Squared Euclidean distance D[n, c] of Key n to centroid c (float32 [N][m]).

    The baseline the article compares against (QVG, "Step 1") gives each Key
    its nearest high-precision centroid. The pages fix no arithmetic for it;
    the reading taken mirrors the QSAC objective's structure so that the same
    kernels can evaluate either: r = k - c in float32; per group G a running
    sum p_G = t_0 + t_1 + ... + t_{g-1} of t_j = r_j * r_j taken channel by
    channel in ascending order (no fused multiply-add); then
    D = ((p_0 + p_1) + p_2) + ... left to right.
    """
    k = np.asarray(k, dtype=F32)
    C = np.asarray(C, dtype=F32)
    N, d = k.shape
    nG = d // g
    D = None
    for G in range(nG):
        p = None
        for j in range(G * g, (G + 1) * g):
            r = k[:, None, j] - C[None, :, j]
            t = r * r
            p = t if p is None else p + t
        D = p if D is None else D + p
    assert D is not None and D.shape == (N, C.shape[0])
    return D


def nearest_assign32(k: np.ndarray, C: np.ndarray, g: int, chunk: int = 2048) -> np.ndarray:
    """QVG's rule: argmin_c of ``nearest_objective``, ties to the smallest id."""
    k = np.asarray(k, dtype=F32)
    out = np.empty(k.shape[0], np.int64)
    for a in range(0, k.shape[0], chunk):
        out[a:a + chunk] = np.argmin(nearest_objective(k[a:a + chunk], C, g), axis=1)
    return out


def postq_objective(k: np.ndarray, C: np.ndarray, S: np.ndarray, g: int) -> np.ndarray:
    """Sensitivity-weighted error left after the actual INT2 quantization
    (float32 [N][m]): the "exact post-rounding error" alternative to the
    range form of the QSAC objective.

    "Step 1" of the article says the nearest centroid is not necessarily the
    best one once the residual is quantized; instead of the range proxy this
    variant quantizes the residual r = k - c with the cache's own per-group
    INT2 (``int2_quantize``, ``int2_dequant``) and scores
    J = sum_G S_G * E_G, E_G = sum over j in G of (r_j - rhat_j)^2,
    in float32: per group the running sum E = t_0 + t_1 + ... of
    t_j = e_j * e_j, e_j = r_j - rhat_j, channels in ascending order; then
    u_G = S_G * E_G and J = ((u_0 + u_1) + u_2) + ... left to right.
    """
    k = np.asarray(k, dtype=F32)
    C = np.asarray(C, dtype=F32)
    S = np.asarray(S, dtype=F32)
    N, d = k.shape
    m = C.shape[0]
    nG = d // g
    J = np.empty((N, m), F32)
    for c in range(m):
        r = k - C[c][None, :]
        codes, zp, sc = int2_quantize(r, g)
        e = r - int2_dequant(codes, zp, sc, g)
        Jc = None
        for G in range(nG):
            E = None
            for j in range(G * g, (G + 1) * g):
                t = e[:, j] * e[:, j]
                E = t if E is None else E + t
            u = S[G] * E
            Jc = u if Jc is None else Jc + u
        J[:, c] = Jc
    return J


OBJECTIVES = ("qsac", "nearest", "postq")


def objective_values(k, C, S, g: int, objective: str) -> np.ndarray:
    """Assignment cost matrix of the chosen rule (float32 [N][m])."""
    if objective == "qsac":
        return qsac_objective(k, C, S, g)
    if objective == "nearest":
        return nearest_objective(k, C, g)
    if objective == "postq":
        return postq_objective(k, C, S, g)
    raise ValueError(objective)


def assign(k, C, S, g: int, objective: str = "qsac") -> np.ndarray:
    """Centroid id per Key under the chosen rule (QSAC, QVG's nearest centroid,
    or the post-rounding error); ties to the smallest id."""
    if objective == "qsac":
        return qsac_assign(k, C, S, g)
    if objective == "nearest":
        return nearest_assign32(k, C, g)
    if objective == "postq":
        k = np.asarray(k, dtype=F32)
        out = np.empty(k.shape[0], np.int64)
        for a in range(0, k.shape[0], 2048):
            out[a:a + 2048] = np.argmin(postq_objective(k[a:a + 2048], C, S, g), axis=1)
        return out
    raise ValueError(objective)


# ---------------------------------------------------------------------------
# O4 / O5 -- per-group asymmetric INT2
# ---------------------------------------------------------------------------

def int2_quantize(x: np.ndarray, g: int):
    """Per-token, per-group asymmetric 2-bit quantization of x [N][d] (float32).

    "Step 1" quantizes the Key-centroid residual to 2 bits; Values use plain
    per-group INT2 (no centroid). The quantizer is the min/max asymmetric one:
    for each group, mn and mx of the values (signed zeros folded to +0);
    zero-point zp = the largest float16 <= mn; step scale = the smallest
    float16 >= (mx - zp) / 3 (float32 correctly rounded divide) whose triple
    is a float16 as well (``fp16_step_up``); codes
    c_j = min(max(rint((x_j - zp) / scale), 0), 3) with rint ties-to-even and
    zp, scale taken as the float32 values of the stored float16; a zero step
    gives all-zero codes. Directed rounding of the stored parameters keeps the
    stored grid [zp, zp + 3 scale] covering [mn, mx], and the step rule makes
    each offset code * scale exactly a float16 value.

    Returns (codes u8 [N][d], zp f16 [N][nG], scale f16 [N][nG]).
    """
    x = np.asarray(x, dtype=F32)
    N, d = x.shape
    nG = d // g
    xg = x.reshape(N, nG, g)
    mn = xg.min(axis=2) + ZERO32
    mx = xg.max(axis=2) + ZERO32
    zp = fp16_round_down(mn)
    zpf = zp.astype(F32)
    step32 = (mx - zpf) / THREE32
    sc = fp16_step_up(step32)
    scf = sc.astype(F32)
    num = xg - zpf[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = num / scf[:, :, None]
    y = np.where(scf[:, :, None] == 0, ZERO32, y)
    codes = np.clip(np.rint(y), 0, 3).astype(np.uint8)
    return codes.reshape(N, d), zp, sc


def int2_dequant(codes: np.ndarray, zp: np.ndarray, sc: np.ndarray, g: int) -> np.ndarray:
    """float32 reconstruction zp + code * scale (the product is exact)."""
    codes = np.asarray(codes)
    N, d = codes.shape
    nG = d // g
    cg = codes.reshape(N, nG, g).astype(F32)
    prod = cg * sc.astype(F32)[:, :, None]
    return (zp.astype(F32)[:, :, None] + prod).reshape(N, d)


def int2_dequant64(codes, zp, sc, g) -> np.ndarray:
    """Exact (float64) reconstruction zp + code * scale."""
    codes = np.asarray(codes)
    N, d = codes.shape
    nG = d // g
    cg = codes.reshape(N, nG, g).astype(F64)
    return (zp.astype(F64)[:, :, None] + cg * sc.astype(F64)[:, :, None]).reshape(N, d)


# ---------------------------------------------------------------------------
# O7 -- PSAC coefficients
# ---------------------------------------------------------------------------

def psac_coef(k, c, rhat, U) -> np.ndarray:
    """Low-rank record of each Key's remaining error (float16 [N][r]).

    "Step 2" and the PSAC sentence of the abstract: the Key error left after
    quantization is kept along the dominant Query directions. With stored
    values, e = k - (c + rhat) in float32 (first the sum, then the
    difference), and coef = U_r^T e in float64, rounded once to float16.
    """
    k = np.asarray(k, dtype=F32)
    t = np.asarray(c, dtype=F32) + np.asarray(rhat, dtype=F32)
    e = k - t
    coef = e.astype(F64) @ np.asarray(U, dtype=F64)
    return f64_to_fp16(coef)


# ---------------------------------------------------------------------------
# O2-O8 -- quantize-on-insert of a block of tokens (one head)
# ---------------------------------------------------------------------------

def quantize_tokens(k, v, C, S, U, g: int, objective: str = "qsac") -> dict:
    """Everything the cache stores for each token of one head, given one epoch's
    calibration (centroids C [m][d], sensitivity S [nG], basis U [d][r]).

    ``objective`` picks the centroid rule ("qsac", or "nearest" for the QVG
    baseline). A basis with r = 0 columns turns PSAC off: no coefficients are
    stored. Each token's record depends only on the token and the
    calibration, so appending in one call or frame by frame gives the same
    bits.
    """
    k = np.asarray(k, dtype=F32)
    v = np.asarray(v, dtype=F32)
    C = np.asarray(C, dtype=F32)
    ids = assign(k, C, S, g, objective)
    c = C[ids]
    r = k - c
    kcode, kzp, ksc = int2_quantize(r, g)
    rhat = int2_dequant(kcode, kzp, ksc, g)
    coef = psac_coef(k, c, rhat, U)
    vcode, vzp, vsc = int2_quantize(v, g)
    return dict(ids=ids.astype(np.uint8), kcode=kcode, kzp=kzp, kscale=ksc,
                vcode=vcode, vzp=vzp, vscale=vsc, coef=coef)


# ---------------------------------------------------------------------------
# O3 -- centroid construction
# ---------------------------------------------------------------------------

def init_centroids(keys: np.ndarray, m: int) -> np.ndarray:
    """Deterministic seeding: centroid i starts as Key floor(i * N / m)."""
    keys = np.asarray(keys, dtype=F32)
    N = keys.shape[0]
    idx = (np.arange(m, dtype=np.int64) * N) // m
    return keys[idx].copy()


def build_centroids(keys, S, m: int, g: int, iters: int, dtype: str, objective: str = "qsac") -> np.ndarray:
    """Centroid table C [m][d] (float32 values in the stored dtype).

    The article clusters the Keys around high-precision centers ("Step 1";
    the compression figure, "Figure 4", counts the centers as stored
    overhead). The pages give no clustering details; the reading taken is
    Lloyd's algorithm with the QSAC assignment: start from
    ``init_centroids``, then ``iters`` times assign every Key by
    ``qsac_assign`` and replace each centroid by the float64 mean of its
    Keys rounded once to the stored dtype; a centroid with no Keys keeps its
    value. With objective "nearest" (the QVG baseline) the assignment is the
    nearest centroid instead and everything else is the same.
    """
    keys = np.asarray(keys, dtype=F32)
    C = init_centroids(keys, m)
    for _ in range(iters):
        ids = assign(keys, C, S, g, objective)
        for i in range(m):
            sel = keys[ids == i]
            if sel.shape[0]:
                mean = sel.astype(F64).sum(axis=0) / F64(sel.shape[0])
                C[i] = f64_to_storage(mean, dtype)
    return C


def mean_objective(keys, C, S, g, objective: str = "qsac") -> float:
    """Mean over Keys of the smallest assignment cost (float64 of the float32 values)."""
    keys = np.asarray(keys, dtype=F32)
    tot = 0.0
    for a in range(0, keys.shape[0], 2048):
        J = objective_values(keys[a:a + 2048], C, S, g, objective)
        tot += float(J.min(axis=1).astype(F64).sum())
    return tot / keys.shape[0]


# ---------------------------------------------------------------------------
# Canonical packed layout
# ---------------------------------------------------------------------------

def pack2(codes: np.ndarray) -> np.ndarray:
    """Pack 2-bit codes [N][d] into bytes [N][d/4]: channel 4b+t in bits 2t..2t+1 of byte b."""
    c = np.asarray(codes, dtype=np.uint8)
    N, d = c.shape
    c4 = c.reshape(N, d // 4, 4)
    return (c4[:, :, 0] | (c4[:, :, 1] << 2) | (c4[:, :, 2] << 4) | (c4[:, :, 3] << 6)).astype(np.uint8)


def unpack2(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    N, nb = p.shape
    out = np.empty((N, nb, 4), np.uint8)
    for t in range(4):
        out[:, :, t] = (p >> (2 * t)) & 3
    return out.reshape(N, nb * 4)


def bytes_per_token_head(d: int, g: int, r: int) -> int:
    """Packed bytes one token of one head occupies: K and V codes, K and V
    (zero-point, scale) float16 pairs per group, a u8 centroid id and r
    float16 PSAC coefficients."""
    return 2 * (d // 4) + 2 * (d // g) * 4 + 1 + 2 * r


def table_bytes_per_head_epoch(d: int, g: int, m: int, r: int, centroid_bytes: int) -> int:
    """Calibration bytes per head and epoch: centroid table, S_G (float32), U_r (float32)."""
    return m * d * centroid_bytes + (d // g) * 4 + d * r * 4


def compression_ratio(n_tokens: int, d: int, g: int, m: int, r: int, centroid_bytes: int,
                      n_epochs: int = 1) -> float:
    """Compression versus a bf16 K+V cache, counting every stored overhead
    (centroids, quantization parameters, compensation data), as the article's
    compression figure does."""
    bf16 = n_tokens * 2 * d * 2
    packed = n_tokens * bytes_per_token_head(d, g, r) + n_epochs * table_bytes_per_head_epoch(d, g, m, r, centroid_bytes)
    return bf16 / packed


# ---------------------------------------------------------------------------
# O9 -- attention over the compressed cache
# ---------------------------------------------------------------------------

class HeadCache:
    """One head's cache as the oracle sees it: per-token records plus the
    calibration of every epoch and the token at which each epoch starts."""

    def __init__(self, g: int, dtype: str, objective: str = "qsac"):
        self.g = g
        self.dtype = dtype
        self.objective = objective
        self.records = []  # list of (start, record dict)
        self.epochs = []  # list of (start, C, S, U)
        self.length = 0

    def add_epoch(self, C, S, U):
        if self.epochs and self.epochs[-1][0] == self.length:
            self.epochs.pop()  # an epoch that holds no tokens is replaced
        self.epochs.append((self.length, np.asarray(C, F32), np.asarray(S, F32), np.asarray(U, F32)))

    def append(self, k, v):
        if not self.epochs:
            raise RuntimeError("no committed epoch")
        _, C, S, U = self.epochs[-1]
        rec = quantize_tokens(k, v, C, S, U, self.g, self.objective)
        rec["epoch"] = np.full(len(rec["ids"]), len(self.epochs) - 1, np.int64)
        self.records.append((self.length, rec))
        self.length += len(rec["ids"])

    def field(self, name):
        return np.concatenate([r[name] for _, r in self.records], axis=0)

    def khat64(self):
        """Dequantized Keys c_id + zp + code * scale, exact in float64."""
        ids = self.field("ids").astype(np.int64)
        ep = self.field("epoch")
        c = np.empty((len(ids), self.epochs[0][1].shape[1]), F64)
        for e, (_, C, _, _) in enumerate(self.epochs):
            sel = ep == e
            c[sel] = C[ids[sel]].astype(F64)
        return c + int2_dequant64(self.field("kcode"), self.field("kzp"), self.field("kscale"), self.g)

    def vhat64(self):
        return int2_dequant64(self.field("vcode"), self.field("vzp"), self.field("vscale"), self.g)


def cache_logits(q, cache: HeadCache, scale: float) -> np.ndarray:
    """Compensated logits of Queries q [Nq][d] against every cached token.

    The abstract names the quantity to preserve: the attention logits QK^T.
    PSAC adds the stored low-rank Key error back to them: for token j of epoch
    e(j), l_ij = (q_i . khat_j + (q_i U^(e(j))) . coef_j) * scale, in float64.
    """
    q = np.asarray(q, dtype=F64)
    kh = cache.khat64()
    coef = cache.field("coef").astype(F64)
    ep = cache.field("epoch")
    ell = q @ kh.T
    for e, (_, _, _, U) in enumerate(cache.epochs):
        sel = np.nonzero(ep == e)[0]
        if len(sel):
            qu = q @ U.astype(F64)
            ell[:, sel] += qu @ coef[sel].T
    return ell * F64(scale)


def attend(q, cache: HeadCache, k_self=None, v_self=None, mask: str = "none",
           scale: float = None) -> np.ndarray:
    """Attention output of one head (float64 [Nq][d]).

    Every cached token is in the past of the attending chunk (block-causal),
    so all of them are visible. An optional self segment holds the chunk's
    own full-precision K/V; mask "full" lets every Query see all of it,
    "causal" lets Query i see self tokens 0..i. Softmax over all visible
    logits in float64 (max subtracted), output sum_j p_ij vhat_j. Default
    scale 1/sqrt(d).
    """
    q = np.asarray(q, dtype=F64)
    d = q.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    parts_l = []
    parts_v = []
    if cache.length:
        parts_l.append(cache_logits(q, cache, scale))
        parts_v.append(cache.vhat64())
    if k_self is not None and mask != "none" and len(k_self):
        ls = (q @ np.asarray(k_self, F64).T) * F64(scale)
        if mask == "causal":
            nq, ns = ls.shape
            ls = np.where(np.arange(ns)[None, :] <= np.arange(nq)[:, None], ls, -np.inf)
        parts_l.append(ls)
        parts_v.append(np.asarray(v_self, F64))
    ell = np.concatenate(parts_l, axis=1)
    vv = np.concatenate(parts_v, axis=0)
    mrow = ell.max(axis=1, keepdims=True)
    p = np.exp(ell - mrow)
    p /= p.sum(axis=1, keepdims=True)
    return p @ vv


# ---------------------------------------------------------------------------
# Table 1 diagnostic -- top-scoring historical token
# ---------------------------------------------------------------------------

def top1_cached(q, cache: HeadCache) -> np.ndarray:
    """Per Query, the cached token with the largest compensated logit
    q . khat_j + (q U^(e(j))) . coef_j (float64; the first index on a tie)."""
    return np.argmax(cache_logits(q, cache, 1.0), axis=1)


def top1_dense(q, k) -> np.ndarray:
    """Per Query, the token with the largest full-precision logit q . k_j
    (float64; the first index on a tie)."""
    return np.argmax(np.asarray(q, F64) @ np.asarray(k, F64).T, axis=1)


def top1_change_rate(q, k_full, cache: HeadCache) -> float:
    """The article's attention analysis ("Table 1"): how often the top-scoring
    historical token of a Query differs between the quantized cache and full
    precision, as a fraction of Queries."""
    return float(np.mean(top1_cached(q, cache) != top1_dense(q, k_full)))
