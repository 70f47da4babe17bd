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
// The eigensolve is a cyclic two-sided Jacobi method run by one workgroup per
// head. Each round applies d/2 disjoint plane rotations chosen by a
// round-robin (tournament) pairing, so every rotation of a round is
// independent: the workgroup updates A (float64, packed upper triangle in
// LDS) as 2x2 blocks B' = R_a^T B R_b and accumulates V (float32 in LDS).
// A 128x128 head fits in 130 KB of the 160 KB LDS of a CDNA4 CU, so the whole
// solve runs without leaving the CU.
#include "qwm_dev.h"
#include "qwm_internal.h"

namespace qwm {

namespace {

// Gram rows [16*rb, 16*rb + 16) of one head, float64 accumulation of exact
// products (bf16 and fp32 products are exact in float64).
template <int D, int DT>
__global__ __launch_bounds__(256) void gram_kernel(const void* q, int64_t n, double* gram) {
  constexpr int CPT = D / 16;  // columns per thread
  constexpr int ROWS = 64;
  __shared__ float qs[ROWS][D + 1];
  const int rb = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int il = tid >> 4, jc = tid & 15;
  const int i = rb * 16 + il;
  double acc[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) acc[k] = 0.0;
  for (int64_t t0 = 0; t0 < n; t0 += ROWS) {
    const int rows = (int)((n - t0) < ROWS ? (n - t0) : ROWS);
    __syncthreads();
    for (int e = tid; e < ROWS * D; e += 256) {
      const int rr = e / D, cc = e % D;
      qs[rr][cc] = (rr < rows) ? load_in<DT>(q, ((int64_t)h * n + t0 + rr) * D + cc) : 0.0f;
    }
    __syncthreads();
    for (int tt = 0; tt < rows; ++tt) {
      const double qi = (double)qs[tt][i];
#pragma unroll
      for (int k = 0; k < CPT; ++k) acc[k] = fma(qi, (double)qs[tt][jc + 16 * k], acc[k]);
    }
  }
  double* G = gram + (int64_t)h * D * D;
#pragma unroll
  for (int k = 0; k < CPT; ++k) G[(int64_t)i * D + jc + 16 * k] = acc[k];
}

__device__ __forceinline__ int tri_index(int i, int j, int n) {  // i <= j
  return i * n - (i * (i - 1)) / 2 + (j - i);
}
__device__ __forceinline__ int tri(int i, int j, int n) { return i <= j ? tri_index(i, j, n) : tri_index(j, i, n); }

// Player at position pos in round `round` of the tournament ordering:
// position 0 is fixed, the others rotate.
__device__ __forceinline__ int player(int pos, int round, int n) {
  return pos == 0 ? 0 : 1 + (pos - 1 + round) % (n - 1);
}

constexpr int kEigThreads = 512;
constexpr int kMaxSweeps = 30;

template <int N>
__global__ __launch_bounds__(kEigThreads) void eigen_kernel(const double* gram, int64_t n_hist, int r, float* U,
                                                            float* S) {
  constexpr int P = N / 2;
  constexpr int TRI = N * (N + 1) / 2;
  constexpr int NW = kEigThreads / 64;
  __shared__ double A[TRI];
  __shared__ float V[N * N];
  __shared__ double rc[P], rs[P], rt[P];
  __shared__ int rp[P], rq[P];
  __shared__ double red_off[NW], red_diag[NW];
  __shared__ int sel[kRankPad];
  __shared__ int done;

  const int h = blockIdx.x, tid = threadIdx.x;
  const double* G = gram + (int64_t)h * N * N;
  for (int idx = tid; idx < N * N; idx += kEigThreads) {
    const int i = idx / N, j = idx % N;
    if (i <= j) A[tri_index(i, j, N)] = G[idx];
    V[idx] = (i == j) ? 1.0f : 0.0f;
  }
  // Sensitivity from the Gram diagonal: S_G = (sum_{j in G} Gram_jj) / M.
  if (tid < N / kGroup) {
    double s = 0.0;
    for (int j = tid * kGroup; j < (tid + 1) * kGroup; ++j) s += G[(int64_t)j * N + j];
    S[h * (N / kGroup) + tid] = (float)(s / (double)n_hist);
  }
  __syncthreads();

  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    // Convergence: off-diagonal energy relative to the diagonal.
    double off = 0.0, dg = 0.0;
    for (int i = tid; i < N; i += kEigThreads) {
      const double d = A[tri_index(i, i, N)];
      dg += d * d;
      for (int j = i + 1; j < N; ++j) {
        const double x = A[tri_index(i, j, N)];
        off += x * x;
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      off += __shfl_xor(off, o);
      dg += __shfl_xor(dg, o);
    }
    if ((tid & 63) == 0) {
      red_off[tid >> 6] = off;
      red_diag[tid >> 6] = dg;
    }
    __syncthreads();
    if (tid == 0) {
      double so = 0.0, sd = 0.0;
      for (int w = 0; w < NW; ++w) {
        so += red_off[w];
        sd += red_diag[w];
      }
      done = (so <= 1e-26 * sd) ? 1 : 0;
    }
    __syncthreads();
    if (done) break;

    for (int round = 0; round < N - 1; ++round) {
      if (tid < P) {
        const int a = player(tid, round, N), b = player(N - 1 - tid, round, N);
        const int p = a < b ? a : b, q = a < b ? b : a;
        const double app = A[tri_index(p, p, N)], aqq = A[tri_index(q, q, N)], apq = A[tri_index(p, q, N)];
        double c = 1.0, s = 0.0, t = 0.0;
        if (apq != 0.0) {
          const double tau = (aqq - app) / (2.0 * apq);
          t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
        }
        rp[tid] = p;
        rq[tid] = q;
        rc[tid] = c;
        rs[tid] = s;
        rt[tid] = t;
      }
      __syncthreads();
      // A <- J^T A J as 2x2 blocks over pairs (a <= b); every element of A
      // belongs to exactly one block, so threads never touch the same entry.
      for (int bi = tid; bi < P * P; bi += kEigThreads) {
        const int a = bi / P, b = bi % P;
        if (a > b) continue;
        const int pa = rp[a], qa = rq[a];
        if (a == b) {
          const double t = rt[a];
          if (t != 0.0) {
            const int ip = tri_index(pa, pa, N), iq = tri_index(qa, qa, N), ipq = tri_index(pa, qa, N);
            const double apq = A[ipq];
            A[ip] = A[ip] - t * apq;
            A[iq] = A[iq] + t * apq;
            A[ipq] = 0.0;
          }
          continue;
        }
        const int pb = rp[b], qb = rq[b];
        const double ca = rc[a], sa = rs[a], cb = rc[b], sb = rs[b];
        const int i11 = tri(pa, pb, N), i12 = tri(pa, qb, N), i21 = tri(qa, pb, N), i22 = tri(qa, qb, N);
        const double x11 = A[i11], x12 = A[i12], x21 = A[i21], x22 = A[i22];
        const double y11 = ca * x11 - sa * x21, y12 = ca * x12 - sa * x22;
        const double y21 = sa * x11 + ca * x21, y22 = sa * x12 + ca * x22;
        A[i11] = cb * y11 - sb * y12;
        A[i12] = sb * y11 + cb * y12;
        A[i21] = cb * y21 - sb * y22;
        A[i22] = sb * y21 + cb * y22;
      }
      // V <- V J (columns p, q of every row).
      for (int vi = tid; vi < P * N; vi += kEigThreads) {
        const int pr = vi % P, row = vi / P;
        const float c = (float)rc[pr], s = (float)rs[pr];
        const int p = rp[pr], q = rq[pr];
        const float vp = V[row * N + p], vq = V[row * N + q];
        V[row * N + p] = c * vp - s * vq;
        V[row * N + q] = s * vp + c * vq;
      }
      __syncthreads();
    }
  }

  // Top-r eigenvalues (descending, lowest index on ties) and sign rule.
  if (tid == 0) {
    for (int k = 0; k < r; ++k) {
      int bi = -1;
      double bv = 0.0;
      for (int i = 0; i < N; ++i) {
        bool taken = false;
        for (int kk = 0; kk < k; ++kk) taken |= (sel[kk] == i);
        if (taken) continue;
        const double v = A[tri_index(i, i, N)];
        if (bi < 0 || v > bv) {
          bi = i;
          bv = v;
        }
      }
      sel[k] = bi;
    }
  }
  __syncthreads();
  if (tid < r) {
    const int col = sel[tid];
    int bi = 0;
    float bv = -1.0f;
    for (int i = 0; i < N; ++i) {
      const float v = fabsf(V[i * N + col]);
      if (v > bv) {
        bv = v;
        bi = i;
      }
    }
    rc[tid] = (V[bi * N + col] < 0.0f) ? -1.0 : 1.0;
  }
  __syncthreads();
  for (int idx = tid; idx < N * r; idx += kEigThreads) {
    const int i = idx / r, k = idx % r;
    U[(int64_t)h * N * r + idx] = (float)rc[k] * V[i * N + sel[k]];
  }
}

}  // namespace

hipError_t launch_gram(int D, int dtype, const void* q, int64_t n, int H, double* gram, hipStream_t s) {
  dim3 grid((unsigned)(D / 16), (unsigned)H), block(256);
  if (D == 128 && dtype == 0)
    hipLaunchKernelGGL((gram_kernel<128, 0>), grid, block, 0, s, q, n, gram);
  else if (D == 128)
    hipLaunchKernelGGL((gram_kernel<128, 1>), grid, block, 0, s, q, n, gram);
  else if (dtype == 0)
    hipLaunchKernelGGL((gram_kernel<64, 0>), grid, block, 0, s, q, n, gram);
  else
    hipLaunchKernelGGL((gram_kernel<64, 1>), grid, block, 0, s, q, n, gram);
  return hipGetLastError();
}

hipError_t launch_eigen(int D, const double* gram, int64_t n_hist, int H, int r, float* U, float* S,
                        hipStream_t s) {
  dim3 grid((unsigned)H), block(kEigThreads);
  if (D == 128)
    hipLaunchKernelGGL((eigen_kernel<128>), grid, block, 0, s, gram, n_hist, r, U, S);
  else
    hipLaunchKernelGGL((eigen_kernel<64>), grid, block, 0, s, gram, n_hist, r, U, S);
  return hipGetLastError();
}

}  // namespace qwm
