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

__device__ __forceinline__ double rcp_f64(double x) {
  double r = __builtin_amdgcn_rcp(x);
  return r * fma(-x, r, 2.0);  // one Newton step
}

template <int N>
__global__ __launch_bounds__(kEigThreads) void eigen_kernel(const double* gram, int nchunk, int64_t n_hist, int r,
                                                            float* U, float* S) {
  constexpr int CPT = N / 8;  // columns of A per thread
  __shared__ double Vst[N * N];  // reflector k in row k, columns k+1..N-1
  __shared__ double vv[2][N], pp[2][N];
  __shared__ double dg[N], ev[N], e2[N], betas[N], zbuf[N];
  __shared__ double misc[4];  // lo, hi, tnorm, pivmin

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
#pragma unroll
    for (int u = 0; u < CPT; ++u)
      if (colof(u) == i) zbuf[i] = a[u];
  }
  __syncthreads();
  // Sensitivity from the Gram diagonal: S_G = (sum_{j in G} Gram_jj) / M.
  if (tid < N / kGroup) {
    double sg = 0.0;
    for (int j = tid * kGroup; j < (tid + 1) * kGroup; ++j) sg += zbuf[j];
    S[h * (N / kGroup) + tid] = (float)(sg / (double)n_hist);
  }

  // Reflector of step k from row k (done by the 8 lanes owning row k):
  // x = A[k][k+1..], alpha = -sign(x0)|x|, v = x - alpha e1, beta = 2 / v.v.
  // v is written over the full length with zeros at 0..k, so the product and
  // the update of the step need no masks.
  auto reflector = [&](int k, int buf) {
    if (i == k) {
      double sq = 0.0, x0 = 0.0;
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int j = colof(u);
        x0 += (j == k + 1) ? a[u] : 0.0;
        sq = fma((j > k + 1) ? a[u] : 0.0, a[u], sq);
      }
      sq = group8_sum(sq);
      x0 = group8_sum(x0);
      double alpha = x0, v0 = x0, beta = 0.0;
      if (sq != 0.0) {
        const double nrm = sqrt(fma(x0, x0, sq));
        alpha = x0 >= 0.0 ? -nrm : nrm;
        v0 = x0 - alpha;
        beta = 2.0 / fma(v0, v0, sq);
      }
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int j = colof(u);
        const double v = (j > k + 1) ? a[u] : ((j == k + 1) ? v0 : 0.0);
        vv[buf][j] = v;
        Vst[k * N + j] = v;
        if (j == k) dg[k] = a[u];
      }
      if (c == 0) {
        ev[k] = alpha;
        betas[k] = beta;
      }
    }
  };

  // ---- 1. tridiagonalization, two barriers per step
  reflector(0, 0);
  __syncthreads();
  for (int k = 0; k < N - 2; ++k) {
    const int buf = k & 1;
    const double beta = betas[k];
    if (beta != 0.0) {
      // p = beta * A22 v (rows <= k get p = 0)
      double acc = 0.0;
#pragma unroll
      for (int u = 0; u < CPT; ++u) acc = fma(a[u], vv[buf][colof(u)], acc);
      acc = group8_sum(acc);
      if (row_ok && c == 0) pp[buf][i] = (i > k) ? beta * acc : 0.0;
      __syncthreads();
      // w = p - (beta/2)(p.v) v ; A22 -= v w^T + w v^T
      double t = 0.0;
#pragma unroll
      for (int j = lane; j < N; j += 64) t = fma(pp[buf][j], vv[buf][j], t);
      const double K = 0.5 * beta * wave_sum(t);
      if (row_ok) {
        const double vi = vv[buf][i], wi = fma(-K, vi, pp[buf][i]);
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
          const int j = colof(u);
          const double vj = vv[buf][j], wj = fma(-K, vj, pp[buf][j]);
          a[u] = fma(-vi, wj, fma(-wi, vj, a[u]));
        }
      }
    }
    // the next reflector needs only row k+1, which its owners just updated
    if (k + 1 < N - 2) reflector(k + 1, buf ^ 1);
    __syncthreads();
  }
  if (row_ok && i >= N - 2) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int j = colof(u);
      if (j == i) dg[i] = a[u];
      if (i == N - 2 && j == N - 1) ev[N - 2] = a[u];
    }
  }
  if (tid == 0) {
    ev[N - 1] = 0.0;
    betas[N - 2] = 0.0;
    betas[N - 1] = 0.0;
  }
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

    // ---- 3. inverse iteration: pivoted LU of T - lam I (pivot reciprocals
    // kept), then solves until the growth shows convergence (at most 3).
    const double tol = 2.220446049250313e-16 * tn;
    Dist Ai, Bb, Cc, Dd;  // Ai holds 1 / pivot
    uint64_t piv0 = 0, piv1 = 0;
    double a_cur = dg[0] - lam, b_cur = ev[0];
    for (int k = 0; k < N - 1; ++k) {
      const double ck = ev[k];
      const double a_next = dg[k + 1] - lam;
      const double b_next = (k + 1 < N - 1) ? ev[k + 1] : 0.0;
      double sai, sb, sc, sd;
      if (fabs(a_cur) >= fabs(ck)) {
        if (a_cur == 0.0) a_cur = tol;
        sai = rcp_f64(a_cur);
        const double mult = ck * sai;
        sb = b_cur;
        sc = mult;
        sd = 0.0;
        a_cur = a_next - mult * b_cur;
        b_cur = b_next;
      } else {
        sai = rcp_f64(ck);
        const double mult = a_cur * sai;
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
      Ai.put(k, sai, lane);
      Bb.put(k, sb, lane);
      Cc.put(k, sc, lane);
      Dd.put(k, sd, lane);
    }
    if (a_cur == 0.0) a_cur = tol;
    Ai.put(N - 1, rcp_f64(a_cur), lane);

    y.s0 = 1.0;
    y.s1 = (lane + 64 < N) ? 1.0 : 0.0;
    for (int iter = 0; iter < 3; ++iter) {
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
      double y1 = ycur * Ai.get(N - 1);
      y.put(N - 1, y1, lane);
      double y0 = (y.get(N - 2) - Bb.get(N - 2) * y1) * Ai.get(N - 2);
      y.put(N - 2, y0, lane);
      double y2 = y1;
      y1 = y0;
      for (int k = N - 3; k >= 0; --k) {
        const double yk = (y.get(k) - Bb.get(k) * y1 - Dd.get(k) * y2) * Ai.get(k);
        y.put(k, yk, lane);
        y2 = y1;
        y1 = yk;
      }
      // the start vector had max-norm 1: a growth near 1 / (eps |T|) means lam
      // is an eigenvalue to working precision and y has converged
      const double mx = wave_max(fmax(fabs(y.s0), fabs(y.s1)));
      if (mx > 0.0) {
        const double inv = 1.0 / mx;
        y.s0 *= inv;
        y.s1 *= inv;
      }
      if (mx * tol >= 0.03) break;
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
      const double v0 = Vst[k * N + i0];  // zero at and left of the diagonal
      const double v1 = (i1 < N) ? Vst[k * N + i1] : 0.0;
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
