// PSAC subspace and QSAC sensitivity from historical Queries (gfx950).
//
// Method (QuantWM; roboind.com article "Step 2": the energy of historical
// Queries concentrates in a few principal directions; fugumt.com abstract:
// "dominant Query subspace", "historical Query sensitivity"):
//   Gram = Q^T Q (uncentered, float64),
//   S_G  = (sum over the group's channels of Gram_jj) / M, stored float32,
//   U_r  = eigenvectors of Gram with the r largest eigenvalues, descending,
//          each column's largest-magnitude entry positive (lowest index on ties).
//
// The eigensolve runs in one workgroup per head, entirely in LDS (the
// float64 Gram of a 128-channel head plus work arrays take ~140 KB of the
// 160 KB of a CDNA4 CU): Householder tridiagonalization, multisection for the
// r largest eigenvalues, inverse iteration, Gram-Schmidt and
// back-transformation (see eigen_kernel).
#include "qwm_dev.h"
#include "qwm_internal.h"

namespace qwm {

namespace {

// Partial Gram of one head: block (32x32 tile, head, token chunk), float64
// accumulation of exact products (bf16 and fp32 products are exact in
// float64). The eigensolver adds the chunk partials in chunk order.
template <int D, int DT>
__global__ __launch_bounds__(256) void gram_kernel(const void* q, int64_t n, int nchunk, double* gram) {
  constexpr int NT = D / 32;
  constexpr int ROWS = 64;
  __shared__ float qa[ROWS][33], qb[ROWS][33];
  const int tile = blockIdx.x, h = blockIdx.y, mc = blockIdx.z, tid = threadIdx.x;
  const int ti = tile / NT, tj = tile % NT;
  const int i = tid >> 3, jq = tid & 7;  // row i of the tile, columns jq + 8u
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  const int64_t ta = n * mc / nchunk, tb = n * (mc + 1) / nchunk;
  for (int64_t t0 = ta; t0 < tb; t0 += ROWS) {
    const int rows = (int)((tb - t0) < ROWS ? (tb - t0) : ROWS);
    __syncthreads();
    for (int e = tid; e < ROWS * 32; e += 256) {
      const int rr = e / 32, cc = e % 32;
      const int64_t base = ((int64_t)h * n + t0 + rr) * D;
      qa[rr][cc] = (rr < rows) ? load_in<DT>(q, base + 32 * ti + cc) : 0.0f;
      qb[rr][cc] = (rr < rows) ? load_in<DT>(q, base + 32 * tj + cc) : 0.0f;
    }
    __syncthreads();
    for (int tt = 0; tt < rows; ++tt) {
      const double av = (double)qa[tt][i];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] = fma(av, (double)qb[tt][jq + 8 * u], acc[u]);
    }
  }
  double* G = gram + ((int64_t)h * nchunk + mc) * D * D;
#pragma unroll
  for (int u = 0; u < 4; ++u) G[(int64_t)(32 * ti + i) * D + 32 * tj + jq + 8 * u] = acc[u];
}

// ---------------------------------------------------------------- eigensolver
//
// Top-r eigenpairs of one head's float64 Gram, one 1024-thread workgroup per
// head, everything in LDS:
//  1. Householder tridiagonalization T = Q^T G Q (126 steps for d = 128; per
//     step one wave forms the reflector, all 16 waves do the matrix-vector
//     product and the symmetric rank-2 update). Reflector k is kept in row k
//     of A, right of the diagonal.
//  2. Wave w finds the w-th largest eigenvalue of T by multisection: its 64
//     lanes evaluate Sturm counts at 64 points of the current interval.
//  3. Wave w computes the eigenvector of T by inverse iteration with a
//     pivoted tridiagonal LU; the serial recurrences run wave-uniformly with
//     the length-d arrays held two elements per lane (readlane to fetch).
//  4. Modified Gram-Schmidt across the r vectors (descending eigenvalues),
//     back-transformation u = H_0 ... H_{d-3} z, sign rule.

__device__ __forceinline__ double readlane_f64(double x, int l) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), l);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), l);
  return __hiloint2double(hi, lo);
}

// A length-N array held by one wave, element k in lane k % 64, slot k / 64.
struct Dist {
  double s0 = 0.0, s1 = 0.0;
  __device__ __forceinline__ double get(int k) const { return readlane_f64(k < 64 ? s0 : s1, k & 63); }
  __device__ __forceinline__ void put(int k, double v, int lane) {
    if (lane == (k & 63)) {
      if (k < 64)
        s0 = v;
      else
        s1 = v;
    }
  }
};

constexpr int kEigThreads = 1024;

template <int N>
__global__ __launch_bounds__(kEigThreads) void eigen_kernel(const double* gram, int nchunk, int64_t n_hist, int r,
                                                            float* U, float* S) {
  constexpr int LDA = N + 1;  // padded pitch: rows start on different banks
  __shared__ double A[N * LDA];
  __shared__ double dg[N], ev[N], e2[N], betas[N], vv[N], pp[N], zbuf[N];
  __shared__ double misc[4];  // lo, hi, tnorm, pivmin

  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const double* G = gram + (int64_t)h * nchunk * N * N;
  for (int idx = tid; idx < N * N; idx += kEigThreads) {
    double x = G[idx];
    for (int c = 1; c < nchunk; ++c) x += G[(int64_t)c * N * N + idx];  // chunk order
    A[(idx / N) * LDA + idx % N] = x;
  }
  __syncthreads();
  // Sensitivity from the Gram diagonal: S_G = (sum_{j in G} Gram_jj) / M.
  if (tid < N / kGroup) {
    double s = 0.0;
    for (int j = tid * kGroup; j < (tid + 1) * kGroup; ++j) s += A[j * LDA + j];
    S[h * (N / kGroup) + tid] = (float)(s / (double)n_hist);
  }

  // ---- 1. tridiagonalization
  for (int k = 0; k < N - 2; ++k) {
    const int m = N - 1 - k;  // length of the reflector
    double* rowk = A + k * LDA + k + 1;
    if (wave == 0) {
      const double x0 = rowk[0];
      double s = 0.0;
      for (int j = 1 + lane; j < m; j += 64) s += rowk[j] * rowk[j];
      s = wave_sum(s);
      double alpha = x0, v0 = x0, beta = 0.0;
      if (s != 0.0) {
        const double nrm = sqrt(x0 * x0 + s);
        alpha = x0 >= 0.0 ? -nrm : nrm;
        v0 = x0 - alpha;
        beta = 2.0 / (v0 * v0 + s);
      }
      for (int j = lane; j < m; j += 64) vv[j] = (j == 0) ? v0 : rowk[j];
      if (lane == 0) {
        dg[k] = A[k * LDA + k];
        ev[k] = alpha;
        betas[k] = beta;
        rowk[0] = v0;
      }
    }
    __syncthreads();
    const double beta = betas[k];
    if (beta != 0.0) {
      // p = beta * A22 v: 8 threads per row; thread c owns columns 8c..8c+7 and
      // 64+8c..64+8c+7, so the 8 rows x 8 chunks of a wave hit distinct bank
      // pairs (row pitch 129 doubles = 2 banks mod 64).
      const int i = tid >> 3, c = tid & 7;
      double acc = 0.0;
      if (i < m) {
        const double* row = A + (k + 1 + i) * LDA + k + 1;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int j = (jj < 8) ? (8 * c + jj) : (64 + 8 * c + jj - 8);
          if (j < m) acc += row[j] * vv[j];
        }
      }
      acc = group8_sum(acc);
      if (i < m && c == 0) pp[i] = beta * acc;
      __syncthreads();
      // w = p - (beta/2)(p.v) v ; A22 -= v w^T + w v^T
      double t = 0.0;
      for (int j = lane; j < m; j += 64) t += pp[j] * vv[j];
      const double K = 0.5 * beta * wave_sum(t);
      if (i < m) {
        double* row = A + (k + 1 + i) * LDA + k + 1;
        const double vi = vv[i], wi = pp[i] - K * vi;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int j = (jj < 8) ? (8 * c + jj) : (64 + 8 * c + jj - 8);
          if (j < m) {
            const double vj = vv[j], wj = pp[j] - K * vj;
            row[j] = row[j] - (vi * wj + wi * vj);
          }
        }
      }
      __syncthreads();
    }
  }
  if (tid == 0) {
    dg[N - 2] = A[(N - 2) * LDA + N - 2];
    dg[N - 1] = A[(N - 1) * LDA + N - 1];
    ev[N - 2] = A[(N - 2) * LDA + N - 1];
    ev[N - 1] = 0.0;
    betas[N - 2] = 0.0;
    betas[N - 1] = 0.0;
  }
  __syncthreads();
  for (int i = tid; i < N; i += kEigThreads) e2[i] = ev[i] * ev[i];
  if (wave == 0) {
    double lo = __builtin_inf(), hi = -__builtin_inf(), tn = 0.0, emax = 0.0;
    for (int i = lane; i < N; i += 64) {
      const double ri = fabs(ev[i]) + (i > 0 ? fabs(ev[i - 1]) : 0.0);
      lo = fmin(lo, dg[i] - ri);
      hi = fmax(hi, dg[i] + ri);
      tn = fmax(tn, fabs(dg[i]) + ri);
      emax = fmax(emax, ev[i] * ev[i]);
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

  Dist y;
  if (wave < r) {
    // ---- 2. the wave-th largest eigenvalue by 64-way multisection
    const int j = N - 1 - wave;  // ascending index
    double lo = misc[0], hi = misc[1];
    const double tn = misc[2], pivmin = misc[3];
    for (int it = 0; it < 64; ++it) {
      if (hi - lo <= 4.0 * 2.220446049250313e-16 * fmax(fabs(lo), fabs(hi)) + pivmin) break;
      const double x = lo + (hi - lo) * (double)(lane + 1) / 65.0;
      double q = dg[0] - x;
      int cnt = q < 0.0;
      for (int i = 1; i < N; ++i) {
        if (fabs(q) < pivmin) q = -pivmin;
        double rq = __builtin_amdgcn_rcp(q);
        rq = rq * fma(-q, rq, 2.0);  // one Newton step: a count is insensitive to the last bits
        q = (dg[i] - x) - e2[i - 1] * rq;
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

    // ---- 3. inverse iteration: pivoted LU of T - lam I, two solves
    const double tol = 2.220446049250313e-16 * tn;
    Dist Aa, Bb, Cc, Dd;
    uint64_t piv0 = 0, piv1 = 0;
    double a_cur = dg[0] - lam, b_cur = ev[0];
    for (int k = 0; k < N - 1; ++k) {
      const double ck = ev[k];
      const double a_next = dg[k + 1] - lam;
      const double b_next = (k + 1 < N - 1) ? ev[k + 1] : 0.0;
      double sa, sb, sc, sd;
      if (fabs(a_cur) >= fabs(ck)) {
        if (a_cur == 0.0) a_cur = tol;
        const double mult = ck / a_cur;
        sa = a_cur;
        sb = b_cur;
        sc = mult;
        sd = 0.0;
        a_cur = a_next - mult * b_cur;
        b_cur = b_next;
      } else {
        const double mult = a_cur / ck;
        sa = ck;
        sb = a_next;
        sc = mult;
        sd = b_next;
        if (k < 64)
          piv0 |= 1ull << k;
        else
          piv1 |= 1ull << (k - 64);
        a_cur = b_cur - mult * a_next;
        b_cur = -mult * b_next;
      }
      Aa.put(k, sa, lane);
      Bb.put(k, sb, lane);
      Cc.put(k, sc, lane);
      Dd.put(k, sd, lane);
    }
    if (a_cur == 0.0) a_cur = tol;
    Aa.put(N - 1, a_cur, lane);

    y.s0 = 1.0;
    y.s1 = (lane + 64 < N) ? 1.0 : 0.0;
    for (int iter = 0; iter < 2; ++iter) {
      double ycur = y.get(0);
      for (int k = 0; k < N - 1; ++k) {
        const double ynext = y.get(k + 1);
        const double ck = Cc.get(k);
        const bool pk = (k < 64) ? ((piv0 >> k) & 1ull) : ((piv1 >> (k - 64)) & 1ull);
        if (!pk) {
          y.put(k, ycur, lane);
          ycur = ynext - ck * ycur;
        } else {
          y.put(k, ynext, lane);
          ycur = ycur - ck * ynext;
        }
      }
      y.put(N - 1, ycur, lane);
      double y1 = y.get(N - 1) / Aa.get(N - 1);
      y.put(N - 1, y1, lane);
      double y0 = (y.get(N - 2) - Bb.get(N - 2) * y1) / Aa.get(N - 2);
      y.put(N - 2, y0, lane);
      double y2 = y1;
      y1 = y0;
      for (int k = N - 3; k >= 0; --k) {
        const double yk = (y.get(k) - Bb.get(k) * y1 - Dd.get(k) * y2) / Aa.get(k);
        y.put(k, yk, lane);
        y2 = y1;
        y1 = yk;
      }
      const double mx = wave_max(fmax(fabs(y.s0), fabs(y.s1)));
      if (mx > 0.0) {
        y.s0 /= mx;
        y.s1 /= mx;
      }
    }
  }
  __syncthreads();

  // ---- 4a. modified Gram-Schmidt in descending-eigenvalue order
  for (int k = 0; k < r; ++k) {
    if (wave == k) {
      const double nrm = sqrt(wave_sum(y.s0 * y.s0 + y.s1 * y.s1));
      if (nrm > 0.0) {
        y.s0 /= nrm;
        y.s1 /= nrm;
      }
      zbuf[lane] = y.s0;
      if (lane + 64 < N) zbuf[lane + 64] = y.s1;
    }
    __syncthreads();
    if (wave > k && wave < r) {
      const double z0 = zbuf[lane], z1 = (lane + 64 < N) ? zbuf[lane + 64] : 0.0;
      const double dot = wave_sum(y.s0 * z0 + y.s1 * z1);
      y.s0 -= dot * z0;
      y.s1 -= dot * z1;
    }
    __syncthreads();
  }

  if (wave < r) {
    // ---- 4b. back-transformation u = H_0 H_1 ... H_{N-3} z
    for (int k = N - 3; k >= 0; --k) {
      const double beta = betas[k];
      if (beta == 0.0) continue;
      const int i0 = lane, i1 = lane + 64;
      const double v0 = (i0 > k) ? A[k * LDA + i0] : 0.0;
      const double v1 = (i1 > k && i1 < N) ? A[k * LDA + i1] : 0.0;
      const double f = beta * wave_sum(v0 * y.s0 + v1 * y.s1);
      y.s0 -= f * v0;
      y.s1 -= f * v1;
    }
    // ---- sign rule: largest-magnitude entry positive (lowest index on ties)
    double bv = fabs(y.s0);
    int bi = lane;
    if (lane + 64 < N && fabs(y.s1) > bv) {
      bv = fabs(y.s1);
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
    const double pivot = (bi < 64) ? readlane_f64(y.s0, bi) : readlane_f64(y.s1, bi - 64);
    const double sg = pivot < 0.0 ? -1.0 : 1.0;
    float* Uh = U + (int64_t)h * N * r;
    Uh[lane * r + wave] = (float)(sg * y.s0);
    if (lane + 64 < N) Uh[(lane + 64) * r + wave] = (float)(sg * y.s1);
  }
}

}  // namespace

int gram_chunks(int64_t n) {
  int64_t c = (n + 1023) / 1024;
  if (c > kGramMaxChunks) c = kGramMaxChunks;
  if (c < 1) c = 1;
  return (int)c;
}

hipError_t launch_gram(int D, int dtype, const void* q, int64_t n, int H, double* gram, hipStream_t s) {
  const int nchunk = gram_chunks(n);
  dim3 grid((unsigned)((D / 32) * (D / 32)), (unsigned)H, (unsigned)nchunk), block(256);
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

hipError_t launch_eigen(int D, const double* gram, int nchunk, int64_t n_hist, int H, int r, float* U, float* S,
                        hipStream_t s) {
  dim3 grid((unsigned)H), block(kEigThreads);
  if (D == 128)
    hipLaunchKernelGGL((eigen_kernel<128>), grid, block, 0, s, gram, nchunk, n_hist, r, U, S);
  else
    hipLaunchKernelGGL((eigen_kernel<64>), grid, block, 0, s, gram, nchunk, n_hist, r, U, S);
  return hipGetLastError();
}

}  // namespace qwm
