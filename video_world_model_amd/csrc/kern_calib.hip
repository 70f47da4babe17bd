// PSAC subspace and QSAC sensitivity from historical Queries (gfx950).
//
// Method (QuantWM; roboind.com article "Step 2": the energy of historical
// Queries concentrates in a few principal directions; fugumt.com abstract:
// QSAC weighs channels by the sensitivity of historical Queries, PSAC works
// in their dominant subspace):
//   Gram = Q^T Q (uncentered, float64),
//   S_G  = (sum over the group's channels of Gram_jj) / M, stored float32,
//   U_r  = eigenvectors of Gram with the r largest eigenvalues, descending,
//          each column's largest-magnitude entry positive (lowest index on ties).
//
// S_G needs only the Gram's diagonal: diag_kernel forms it (with the same fma
// sequence as the Gram's diagonal entries) on the cache stream, so the k-means
// does not wait for the full Gram, which runs beside the eigensolve.
//
// The eigensolve runs in one workgroup per head (the Gram in registers, the
// float64 reflectors plus work arrays in ~140 KB of the 160 KB of LDS of a
// CDNA4 CU): Householder tridiagonalization, multisection for the
// r largest eigenvalues, inverse iteration, Gram-Schmidt and
// back-transformation (see eigen_kernel).
#include "qwm_dev.h"
#include "qwm_internal.h"

namespace qwm {

namespace {

// Partial Gram of one head: block (64x64 tile, head, token chunk); thread
// (a, b) owns the 4x4 entries rows 4a.., columns 4b.. of the tile. Tokens are
// staged 64 at a time in LDS as float; products of bf16 or fp32 inputs are
// exact in float64 and are accumulated by fma in token order. The eigensolver
// adds the chunk partials in chunk order.
constexpr int kGramRows = 64;
constexpr int kGramChunkMin = 128;  // tokens per chunk before another chunk is opened

template <int D, int DT>
__global__ __launch_bounds__(256) void gram_kernel(const void* q, int64_t n, int nchunk, double* gram) {
  constexpr int NT = D / 64;
  __shared__ float4 qa[kGramRows][16], qb[kGramRows][16];
  const int tile = blockIdx.x, h = blockIdx.y, mc = blockIdx.z, tid = threadIdx.x;
  const int ti = tile / NT, tj = tile % NT;
  const int ra = tid >> 4, cb = tid & 15;
  double acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = 0.0;
  const int64_t ta = n * mc / nchunk, tb = n * (mc + 1) / nchunk;
  for (int64_t t0 = ta; t0 < tb; t0 += kGramRows) {
    const int rows = (int)((tb - t0) < kGramRows ? (tb - t0) : kGramRows);
    __syncthreads();
#pragma unroll
    for (int e = tid; e < kGramRows * 16; e += 256) {
      const int rr = e >> 4, qd = e & 15;
      float4 va = make_float4(0.f, 0.f, 0.f, 0.f), vb = va;
      if (rr < rows) {
        const int64_t base = ((int64_t)h * n + t0 + rr) * D;
        const int64_t ia = base + 64 * ti + 4 * qd, ib = base + 64 * tj + 4 * qd;
        if constexpr (DT == 0) {
          const uint2 pa = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(q) + ia);
          const uint2 pb = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(q) + ib);
          va = make_float4(__uint_as_float(pa.x << 16), __uint_as_float(pa.x & 0xFFFF0000u),
                           __uint_as_float(pa.y << 16), __uint_as_float(pa.y & 0xFFFF0000u));
          vb = make_float4(__uint_as_float(pb.x << 16), __uint_as_float(pb.x & 0xFFFF0000u),
                           __uint_as_float(pb.y << 16), __uint_as_float(pb.y & 0xFFFF0000u));
        } else {
          va = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(q) + ia);
          vb = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(q) + ib);
        }
      }
      qa[rr][qd] = va;
      qb[rr][qd] = vb;
    }
    __syncthreads();
    for (int tt = 0; tt < rows; ++tt) {
      const float4 fa = qa[tt][ra], fb = qb[tt][cb];
      const double av[4] = {(double)fa.x, (double)fa.y, (double)fa.z, (double)fa.w};
      const double bv[4] = {(double)fb.x, (double)fb.y, (double)fb.z, (double)fb.w};
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fma(av[x], bv[y], acc[x][y]);
    }
  }
  double* G = gram + ((int64_t)h * nchunk + mc) * D * D;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    double* row = G + (int64_t)(64 * ti + 4 * ra + x) * D + 64 * tj + 4 * cb;
    *reinterpret_cast<double2*>(row) = make_double2(acc[x][0], acc[x][1]);
    *reinterpret_cast<double2*>(row + 2) = make_double2(acc[x][2], acc[x][3]);
  }
}

// Diagonal of one head's chunk Gram (head, chunk per block): thread j < D
// forms sum_t q_tj^2 by fma in token order, the operations that give the
// Gram's diagonal entries. Tokens are staged in LDS 64 at a time as float;
// the raw words of the next 64 are loaded into registers before the current
// ones are summed.
template <int D, int DT>
__global__ __launch_bounds__(256) void diag_kernel(const void* q, int64_t n, int nchunk, double* diag) {
  constexpr int ESZ = DT == 0 ? 2 : 4;
  constexpr int WPR = D * ESZ / 16;          // 16-byte words per token row
  constexpr int WPT = kGramRows * WPR / 256;  // words per thread per 64 tokens
  __shared__ float qs[kGramRows][D];
  const int h = blockIdx.x, mc = blockIdx.y, tid = threadIdx.x;
  const int64_t ta = n * mc / nchunk, tb = n * (mc + 1) / nchunk;
  const uint4* qh = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(q) + (size_t)h * n * D * ESZ);
  uint4 w[WPT];
  auto load = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int e = i * 256 + tid;
      const int64_t t = t0 + e / WPR < tb ? t0 + e / WPR : tb - 1;  // rows past the chunk: a valid copy, unused
      w[i] = qh[t * WPR + e % WPR];
    }
  };
  double acc = 0.0;
  if (ta < tb) load(ta);
  for (int64_t t0 = ta; t0 < tb; t0 += kGramRows) {
    const int rows = (int)((tb - t0) < kGramRows ? (tb - t0) : kGramRows);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int e = i * 256 + tid;
      float* dst = &qs[e / WPR][(e % WPR) * (16 / ESZ)];
      if constexpr (DT == 0) {
        const uint32_t ww[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          dst[2 * k] = __uint_as_float(ww[k] << 16);
          dst[2 * k + 1] = __uint_as_float(ww[k] & 0xFFFF0000u);
        }
      } else {
        dst[0] = __uint_as_float(w[i].x);
        dst[1] = __uint_as_float(w[i].y);
        dst[2] = __uint_as_float(w[i].z);
        dst[3] = __uint_as_float(w[i].w);
      }
    }
    __syncthreads();
    if (t0 + kGramRows < tb) load(t0 + kGramRows);
    if (tid < D) {
      for (int tt = 0; tt < rows; ++tt) {
        const double x = (double)qs[tt][tid];
        acc = fma(x, x, acc);
      }
    }
  }
  if (tid < D) diag[((int64_t)h * nchunk + mc) * D + tid] = acc;
}

// Sensitivity S_G = (sum over the group's channels of Gram_jj) / M, one
// block per head: thread j adds the chunk partials of Gram_jj in chunk order,
// then thread G adds its group's 32 diagonal entries in channel order.
template <int N>
__global__ __launch_bounds__(N) void sens_kernel(const double* diagp, int nchunk, int64_t n_hist, float* S) {
  __shared__ double diag[N];
  const int h = blockIdx.x, j = threadIdx.x;
  const double* G = diagp + (int64_t)h * nchunk * N + j;
  double x = 0.0;
  for (int ch = 0; ch < nchunk; ++ch) x += G[(int64_t)ch * N];
  diag[j] = x;
  __syncthreads();
  if (j < N / kGroup) {
    double sg = 0.0;
    for (int t = j * kGroup; t < (j + 1) * kGroup; ++t) sg += diag[t];
    S[h * (N / kGroup) + j] = (float)(sg / (double)n_hist);
  }
}

// ---------------------------------------------------------------- eigensolver
//
// Top-r eigenpairs of one head's float64 Gram, one 1024-thread workgroup per
// head:
//  1. Householder tridiagonalization T = Q^T G Q (126 steps for d = 128). The
//     matrix lives in registers (thread t: row t/8, 16 columns); the 8 lanes
//     of row k form reflector k, every thread takes part in the
//     matrix-vector product and the symmetric rank-2 update, and the owners of
//     row k+1 form the next reflector straight after their own update, so a
//     step costs two barriers. Reflectors are kept in LDS for step 4.
//  2. Wave w finds the w-th largest eigenvalue of T by multisection: its 64
//     lanes evaluate Sturm counts at 64 points of the current interval.
//  3. Wave w computes the eigenvector of T from the twisted factorization
//     of T - lambda I (forward and backward pivots, twist at the smallest
//     |gamma|), one pass each way; the serial recurrences run
//     wave-uniformly with their arrays in LDS.
//  4. Modified Gram-Schmidt across the r vectors (descending eigenvalues),
//     back-transformation u = H_0 ... H_{d-3} z, sign rule.

__device__ __forceinline__ double readlane_f64(double x, int l) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), l);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), l);
  return __hiloint2double(hi, lo);
}

constexpr int kEigThreads = 1024;

__device__ __forceinline__ double rcp_f64(double x) {
  double r = __builtin_amdgcn_rcp(x);
  return r * fma(-x, r, 2.0);  // one Newton step
}

// Pivot guard shared by the Sturm count and the factorizations: a pivot of
// magnitude below pivmin is replaced by -pivmin.
__device__ __forceinline__ double guard_pivot(double q, double pivmin) { return fabs(q) < pivmin ? -pivmin : q; }

// Makes the wave's own LDS writes visible to its other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int N>
__global__ __launch_bounds__(kEigThreads) void eigen_kernel(const double* gram, int nchunk, int r, float* U) {
  constexpr int CPT = N / 8;               // columns of A per thread
  constexpr int NV = N * (N - 1) / 2;      // packed reflectors
  __shared__ double Vst[NV];               // reflector k: columns k+1..N-1 at vrow(k)
  __shared__ double xrow[2][N], erow[2][N], pp[2][N];  // rows k and k+1 of A at step k; p
  __shared__ double dg[N], ev[N], e2[N], betas[N], zbuf[N];
  __shared__ double Dp[kRankPad][N], Dm[kRankPad][N];  // twisted-factorization pivots, one row per eigenvalue
  __shared__ double misc[4];               // lo, hi, tnorm, pivmin
  auto vrow = [](int k) { return k * (N - 1) - k * (k - 1) / 2 - k - 1; };  // + j for column j > k

  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Each thread keeps its share of A in registers: row i, 16 (or 8) columns:
  // 8c..8c+7 and 64+8c..64+8c+7, so the 8 threads of a row are 8 aligned
  // lanes and a row reduction is an 8-lane DPP sum.
  const int i = tid >> 3, c = tid & 7;
  const bool row_ok = i < N;
  auto colof = [&](int u) { return u < 8 ? 8 * c + u : 64 + 8 * c + (u - 8); };
  const double* G = gram + (int64_t)h * nchunk * N * N;
  double a[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) a[u] = 0.0;
  if (row_ok) {
    for (int ch = 0; ch < nchunk; ++ch) {  // chunk partials added in chunk order
      const double* Gc = G + (int64_t)ch * N * N + (int64_t)i * N;
#pragma unroll
      for (int u = 0; u < CPT; ++u) a[u] += Gc[colof(u)];
    }
  }

  // ---- 1. Householder tridiagonalization, two barriers per step.
  // Step k: x = A[k][k+1..], alpha = -sign(x0)|x|, v = x - alpha e_{k+1},
  // beta = 2 / v.v = -1 / (alpha v0), p = beta A v,
  // A -= v w^T + w v^T with w = p - (beta/2)(p.v) v, i.e.
  // A -= v p^T + (p - beta (p.v) v) v^T.
  // At the end of step k-1 the owners of row k publish x (entries <= k set
  // to zero) and the diagonal, and the owners of row k+1 publish that row,
  // which by symmetry is column k+1. Every wave then forms the reflector
  // itself, and the products use x in place of v with one correction for the
  // v0 entry: (A v)_i = (A x)_i - alpha A[k+1][i], p.v = p.x - alpha p_{k+1}.
  // The update with x_{k+1} in place of v0 is wrong only in column k+1, which
  // is finished after this step except for the diagonal of row k+1; its
  // owners add the missing w_{k+1} alpha when they publish it.
  // Rows and columns <= k are finished after step k and never read again
  // (x and p are zero there, so they stay as they are); a wave whose 8 rows
  // are all finished skips the step.
  if (row_ok && i == 0) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int j = colof(u);
      xrow[0][j] = (j > 0) ? a[u] : 0.0;
      if (j == 0) dg[0] = a[u];
    }
  }
  if (row_ok && i == 1) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) erow[0][colof(u)] = a[u];
  }
  __syncthreads();
  const int writer = N / 8 - 1;  // owns row N-1, live on every step
  for (int k = 0; k < N - 2; ++k) {
    const int buf = k & 1;
    const bool live = row_ok && (8 * wave + 7 > k);  // wave-uniform
    double xj[CPT];
    double alpha = 0.0, beta = 0.0, xi = 0.0;
    if (live) {
      const double x0 = xrow[buf][k + 1];
      const double xl0 = xrow[buf][lane], xl1 = (lane + 64 < N) ? xrow[buf][lane + 64] : 0.0;
      const double m0 = (lane > k + 1) ? xl0 : 0.0, m1 = (lane + 64 > k + 1) ? xl1 : 0.0;
      double s4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        xj[u] = xrow[buf][colof(u)];
        s4[u & 3] = fma(a[u], xj[u], s4[u & 3]);
      }
      const double ei = erow[buf][i];
      xi = xrow[buf][i];
      const double sq = wave_sum(fma(m0, m0, m1 * m1));
      alpha = x0;
      double v0 = 0.0;
      if (sq != 0.0) {
        const double nrm = sqrt(fma(x0, x0, sq));
        alpha = x0 >= 0.0 ? -nrm : nrm;
        v0 = x0 - alpha;
        beta = -rcp_f64(alpha * v0);
      }
      if (wave == writer) {
        const double vl0 = (lane == k + 1) ? v0 : m0, vl1 = (lane + 64 == k + 1) ? v0 : m1;
        if (lane > k) Vst[vrow(k) + lane] = vl0;
        if (lane + 64 > k && lane + 64 < N) Vst[vrow(k) + lane + 64] = vl1;
        if (lane == 0) {
          ev[k] = alpha;
          betas[k] = beta;
        }
      }
      const double acc = fma(-alpha, ei, group8_sum((s4[0] + s4[1]) + (s4[2] + s4[3])));
      if (c == 0) pp[buf][i] = (i > k) ? beta * acc : 0.0;
    } else if (row_ok && c == 0) {
      pp[buf][i] = 0.0;
    }
    __syncthreads();
    if (live) {
      double t4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int u = 0; u < CPT; ++u) t4[u & 3] = fma(pp[buf][colof(u)], xj[u], t4[u & 3]);
      const double pt = group8_sum((t4[0] + t4[1]) + (t4[2] + t4[3]));
      const double K2 = beta * fma(-alpha, pp[buf][k + 1], pt);
      const double vi = (i == k + 1) ? xi - alpha : xi;
      const double wi = fma(-K2, vi, pp[buf][i]);
      // p is read again below rather than kept from the loop above: holding
      // both copies would exceed the 128 registers a 1,024-thread block allows
      asm volatile("" ::: "memory");
#pragma unroll
      for (int u = 0; u < CPT; ++u) a[u] = fma(-vi, pp[buf][colof(u)], fma(-wi, xj[u], a[u]));
      // publish rows k+1 and k+2 for the next step
      if (i == k + 1) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
          const int j = colof(u);
          xrow[buf ^ 1][j] = (j > k + 1) ? a[u] : 0.0;
          if (j == k + 1) dg[k + 1] = fma(wi, alpha, a[u]);
        }
      }
      if (i == k + 2) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) erow[buf ^ 1][colof(u)] = a[u];
      }
    }
    __syncthreads();
  }
  // dg[N-2] was published by step N-3
  if (row_ok && i >= N - 2) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int j = colof(u);
      if (i == N - 1 && j == N - 1) dg[N - 1] = a[u];
      if (i == N - 2 && j == N - 1) ev[N - 2] = a[u];
    }
  }

  if (tid == 0) ev[N - 1] = 0.0;
  __syncthreads();
  for (int ii = tid; ii < N; ii += kEigThreads) e2[ii] = ev[ii] * ev[ii];
  if (wave == 0) {
    double lo = __builtin_inf(), hi = -__builtin_inf(), tn = 0.0, emax = 0.0;
    for (int ii = lane; ii < N; ii += 64) {
      const double ri = fabs(ev[ii]) + (ii > 0 ? fabs(ev[ii - 1]) : 0.0);
      lo = fmin(lo, dg[ii] - ri);
      hi = fmax(hi, dg[ii] + ri);
      tn = fmax(tn, fabs(dg[ii]) + ri);
      emax = fmax(emax, ev[ii] * ev[ii]);
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    tn = wave_max(tn);
    emax = wave_max(emax);
    if (lane == 0) {
      const double pivmin = 2.2250738585072014e-308 * fmax(1.0, emax);
      const double pad = 4.0 * 2.220446049250313e-16 * tn + pivmin;
      misc[0] = lo - pad;
      misc[1] = hi + pad;
      misc[2] = tn;
      misc[3] = pivmin;
    }
  }
  __syncthreads();

  double y0 = 0.0, y1 = 0.0;  // wave w's vector: entry l in y0 of lane l, entry 64+l in y1
  if (wave < r) {
    // ---- 2. the wave-th largest eigenvalue by 64-way multisection, to an
    // absolute accuracy of a few ulps of |T|
    const int j = N - 1 - wave;  // ascending index
    double lo = misc[0], hi = misc[1];
    const double tn = misc[2], pivmin = misc[3];
    const double tol = 4.0 * 2.220446049250313e-16 * tn + pivmin;
    for (int it = 0; it < 64; ++it) {
      if (hi - lo <= tol) break;
      const double x = lo + (hi - lo) * (double)(lane + 1) / 65.0;
      double q = dg[0] - x;
      int cnt = q < 0.0;
      for (int ii = 1; ii < N; ++ii) {
        q = (dg[ii] - x) - e2[ii - 1] * rcp_f64(guard_pivot(q, pivmin));  // a count is insensitive to the last bits
        cnt += q < 0.0;
      }
      const uint64_t mask = __ballot(cnt > j);
      const int L = mask ? (__ffsll((unsigned long long)mask) - 1) : 64;
      const double nhi = (L < 64) ? readlane_f64(x, L) : hi;
      const double nlo = (L > 0) ? readlane_f64(x, L - 1) : lo;
      lo = nlo;
      hi = nhi;
    }
    const double lam = 0.5 * (lo + hi);

    // ---- 3. eigenvector of T by the twisted factorization of T - lam I:
    // forward pivots D+ (top down) and backward pivots D- (bottom up), twist
    // index t = argmin |D+_t + D-_t - (d_t - lam)|, then z_t = 1,
    // z_i = -(e_i / D+_i) z_{i+1} above t and z_{i+1} = -(e_i / D-_{i+1}) z_i below.
    double* dp = Dp[wave];
    double* dm = Dm[wave];
    double qf = guard_pivot(dg[0] - lam, pivmin), qb = guard_pivot(dg[N - 1] - lam, pivmin);
    if (lane == 0) {
      dp[0] = qf;
      dm[N - 1] = qb;
    }
    for (int st = 1; st < N; ++st) {
      const int ib = N - 1 - st;
      qf = guard_pivot((dg[st] - lam) - e2[st - 1] * rcp_f64(qf), pivmin);
      qb = guard_pivot((dg[ib] - lam) - e2[ib] * rcp_f64(qb), pivmin);
      if (lane == 0) {
        dp[st] = qf;
        dm[ib] = qb;
      }
    }
    wave_lds_sync();
    double best = __builtin_inf();
    int bt = 0;
    for (int t = lane; t < N; t += 64) {
      const double g = fabs(dp[t] + dm[t] - (dg[t] - lam));
      if (g < best) {
        best = g;
        bt = t;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ov = __shfl_xor(best, o);
      const int ot = __shfl_xor(bt, o);
      if (ov < best || (ov == best && ot < bt)) {
        best = ov;
        bt = ot;
      }
    }
    bt = __builtin_amdgcn_readfirstlane(bt);
    wave_lds_sync();
    // z overwrites dp: entry i of dp is read before z_i is stored there
    double zu = 1.0, zd = 1.0;
    for (int st = 1; st < N; ++st) {
      const int iu = bt - st, id = bt + st;
      if (iu >= 0) zu = -(ev[iu] * rcp_f64(dp[iu])) * zu;
      if (id < N) zd = -(ev[id - 1] * rcp_f64(dm[id])) * zd;
      if (lane == 0) {
        if (iu >= 0) dp[iu] = zu;
        if (id < N) dp[id] = zd;
      }
    }
    if (lane == 0) dp[bt] = 1.0;
    wave_lds_sync();
    y0 = dp[lane];
    y1 = (lane + 64 < N) ? dp[lane + 64] : 0.0;
  }
  __syncthreads();

  // ---- 4a. modified Gram-Schmidt in descending-eigenvalue order
  for (int k = 0; k < r; ++k) {
    if (wave == k) {
      const double nrm = sqrt(wave_sum(y0 * y0 + y1 * y1));
      if (nrm > 0.0) {
        y0 /= nrm;
        y1 /= nrm;
      }
      zbuf[lane] = y0;
      if (lane + 64 < N) zbuf[lane + 64] = y1;
    }
    __syncthreads();
    if (wave > k && wave < r) {
      const double z0 = zbuf[lane], z1 = (lane + 64 < N) ? zbuf[lane + 64] : 0.0;
      const double dot = wave_sum(y0 * z0 + y1 * z1);
      y0 -= dot * z0;
      y1 -= dot * z1;
    }
    __syncthreads();
  }

  if (wave < r) {
    // ---- 4b. back-transformation u = H_0 H_1 ... H_{N-3} z
    for (int k = N - 3; k >= 0; --k) {
      const double beta = betas[k];
      const int i0 = lane, i1 = lane + 64;
      // reflector k is zero at and left of the diagonal; indexes are clamped
      // into its stored row before the select
      const double s0 = Vst[vrow(k) + (i0 > k ? i0 : k + 1)];
      const double s1 = Vst[vrow(k) + (i1 > k && i1 < N ? i1 : k + 1)];
      const double v0 = (i0 > k) ? s0 : 0.0;
      const double v1 = (i1 > k && i1 < N) ? s1 : 0.0;
      const double f = beta * wave_sum(v0 * y0 + v1 * y1);
      y0 -= f * v0;
      y1 -= f * v1;
    }
    // ---- sign rule: largest-magnitude entry positive (lowest index on ties)
    double bv = fabs(y0);
    int bi = lane;
    if (lane + 64 < N && fabs(y1) > bv) {
      bv = fabs(y1);
      bi = lane + 64;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    const double pivot = (bi < 64) ? readlane_f64(y0, bi) : readlane_f64(y1, bi - 64);
    const double sg = pivot < 0.0 ? -1.0 : 1.0;
    float* Uh = U + (int64_t)h * N * r;
    Uh[lane * r + wave] = (float)(sg * y0);
    if (lane + 64 < N) Uh[(lane + 64) * r + wave] = (float)(sg * y1);
  }
}

}  // namespace

int gram_chunks(int64_t n) {
  int64_t c = (n + kGramChunkMin - 1) / kGramChunkMin;
  if (c > kGramMaxChunks) c = kGramMaxChunks;
  if (c < 1) c = 1;
  return (int)c;
}

hipError_t launch_gram(int D, int dtype, const void* q, int64_t n, int H, double* gram, hipStream_t s) {
  const int nchunk = gram_chunks(n);
  dim3 grid((unsigned)((D / 64) * (D / 64)), (unsigned)H, (unsigned)nchunk), block(256);
  if (D == 128 && dtype == 0)
    hipLaunchKernelGGL((gram_kernel<128, 0>), grid, block, 0, s, q, n, nchunk, gram);
  else if (D == 128)
    hipLaunchKernelGGL((gram_kernel<128, 1>), grid, block, 0, s, q, n, nchunk, gram);
  else if (dtype == 0)
    hipLaunchKernelGGL((gram_kernel<64, 0>), grid, block, 0, s, q, n, nchunk, gram);
  else
    hipLaunchKernelGGL((gram_kernel<64, 1>), grid, block, 0, s, q, n, nchunk, gram);
  return hipGetLastError();
}

hipError_t launch_diag(int D, int dtype, const void* q, int64_t n, int H, double* diag, hipStream_t s) {
  const int nchunk = gram_chunks(n);
  dim3 grid((unsigned)H, (unsigned)nchunk), block(256);
  if (D == 128 && dtype == 0)
    hipLaunchKernelGGL((diag_kernel<128, 0>), grid, block, 0, s, q, n, nchunk, diag);
  else if (D == 128)
    hipLaunchKernelGGL((diag_kernel<128, 1>), grid, block, 0, s, q, n, nchunk, diag);
  else if (dtype == 0)
    hipLaunchKernelGGL((diag_kernel<64, 0>), grid, block, 0, s, q, n, nchunk, diag);
  else
    hipLaunchKernelGGL((diag_kernel<64, 1>), grid, block, 0, s, q, n, nchunk, diag);
  return hipGetLastError();
}

hipError_t launch_sens(int D, const double* diag, int nchunk, int64_t n_hist, int H, float* S, hipStream_t s) {
  dim3 grid((unsigned)H), block((unsigned)D);
  if (D == 128)
    hipLaunchKernelGGL((sens_kernel<128>), grid, block, 0, s, diag, nchunk, n_hist, S);
  else
    hipLaunchKernelGGL((sens_kernel<64>), grid, block, 0, s, diag, nchunk, n_hist, S);
  return hipGetLastError();
}

hipError_t launch_eigen(int D, const double* gram, int nchunk, int H, int r, float* U, hipStream_t s) {
  dim3 grid((unsigned)H), block(kEigThreads);
  if (D == 128)
    hipLaunchKernelGGL((eigen_kernel<128>), grid, block, 0, s, gram, nchunk, r, U);
  else
    hipLaunchKernelGGL((eigen_kernel<64>), grid, block, 0, s, gram, nchunk, r, U);
  return hipGetLastError();
}

}  // namespace qwm
