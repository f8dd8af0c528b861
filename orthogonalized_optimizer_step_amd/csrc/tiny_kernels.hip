// Gram Newton-Schulz for small matrices in one launch (Dion3 summary,
// 方法 / 核心模块, "Gram Newton-Schulz" bullet: G = X X^T, then per iteration
// P = aI + bG + cG^2, Q <- P Q, and G <- P G P or, at a restart, X <- Q X,
// G <- X X^T, Q <- I; out = Q X).
//
// For matrices whose Gram side m is at most 64 (and long side at most 1024)
// the GEMM phases would be some twenty launches of a tile or three each, so a
// call of only such matrices is bound by launch latency, and beside larger
// ones they would take 256-row tiles for a few rows.  Here one workgroup per matrix
// runs the whole iteration in fp64: the m x m matrices G, P, Q and a temporary
// live in LDS (four 64 x 64 fp64 buffers, 128 KB, plus a 16 KB staging chunk
// for the Gram), the iterate X (m x n, fp64) in two workspace buffers that
// alternate at restarts.
#include <hip/hip_runtime.h>

#include "dion_internal.h"

namespace dion {

constexpr int TINY_M = 64;
constexpr int TINY_N = 1024;
constexpr int TINY_THREADS = 1024;

namespace {

__device__ __forceinline__ double tiny_in(const void* p, size_t e, int fmt) {
  if (fmt == 1) return (double)((const float*)p)[e];
  const uint16_t u = ((const uint16_t*)p)[e];
  if (fmt == 0) return (double)__uint_as_float((uint32_t)u << 16);
  return (double)(float)__builtin_bit_cast(_Float16, u);
}

__device__ __forceinline__ void tiny_out(void* p, size_t e, double v, int fmt) {
  const float f = (float)v;
  if (fmt == 1) {
    ((float*)p)[e] = f;
  } else if (fmt == 0) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    ((uint16_t*)p)[e] = (uint16_t)(u >> 16);
  } else {
    ((uint16_t*)p)[e] = __builtin_bit_cast(uint16_t, (_Float16)f);
  }
}

// the lowest of the four LDS buffers not in use
__device__ __forceinline__ int tiny_free(int x, int y, int z) {
  for (int b = 0; b < 4; ++b)
    if (b != x && b != y && b != z) return b;
  return 3;
}

}  // namespace

// ids: the batch indices of the matrices this launch covers, one workgroup
// each; coef: K triples (a, b, c) in fp64 with the safety factor folded in;
// restarts: bit k-1 set = restart after iteration k.
__global__ __launch_bounds__(TINY_THREADS) void k_tiny_gns(const MatDesc* __restrict__ descs,
                                                           const int* __restrict__ ids,
                                                           const MatScalars* __restrict__ scalars,
                                                           const int* __restrict__ idx,
                                                           const double* __restrict__ coef, int K,
                                                           unsigned long long restarts, int fmt) {
  const int mi = ids[blockIdx.x];
  const MatDesc& d = descs[mi];
  const int m = d.m, n = d.n;
  const int tid = threadIdx.x;
  const double nu2 = scalars[mi].nu2;                // ||S||_F^2 from the selection
  const double s = nu2 > 0.0 ? 1.0 / sqrt(nu2) : 0.0;
  __shared__ double buf[4][TINY_M * TINY_M];          // row-major, ld TINY_M
  double* X = (double*)d.buf[SLOT_X];                 // m x n, ld n
  double* X2 = (double*)d.buf[SLOT_XT0];
  auto src_row = [&](int j) { return idx ? idx[d.sel0 + j] : j; };

  // X = S / nu, oriented so that m <= n (S^T when the block is tall)
  for (int e = tid; e < m * n; e += TINY_THREADS) {
    const int i = e / n, l = e - (e / n) * n;
    const int sr = d.tall ? l : i, sc = d.tall ? i : l;
    X[e] = tiny_in(d.M, (size_t)src_row(sr) * d.C + sc, fmt) * s;
  }
  __syncthreads();

  // G = X X^T from 32-column chunks of X staged transposed in LDS; thread
  // (i0, j) sums rows i0, i0 + 16, i0 + 32, i0 + 48 of column j along the long
  // side in order (so G[i][j] and G[j][i] take the same sum)
  __shared__ double xc[32 * TINY_M];
  auto gram = [&](double* G) {
    const int j = tid & 63, i0 = tid >> 6;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int l0 = 0; l0 < n; l0 += 32) {
      for (int e = tid; e < 32 * TINY_M; e += TINY_THREADS) {
        const int row = e >> 5, k = e & 31;
        xc[k * TINY_M + row] = (row < m && l0 + k < n) ? X[(size_t)row * n + l0 + k] : 0.0;
      }
      __syncthreads();
      if (j < m) {
        for (int k = 0; k < 32; ++k) {
          const double bk = xc[k * TINY_M + j];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] += xc[k * TINY_M + i0 + 16 * r] * bk;
        }
      }
      __syncthreads();
    }
    if (j < m) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (i0 + 16 * r < m) G[(i0 + 16 * r) * TINY_M + j] = acc[r];
    }
    __syncthreads();
  };
  // C = A B (m x m): thread (i0, j) forms rows i0, i0 + 16, i0 + 32, i0 + 48 of
  // column j, sharing each B[k][j] (rows past m are computed from in-bounds
  // LDS and dropped)
  auto mm = [&](double* C, const double* A, const double* B) {
    const int j = tid & 63, i0 = tid >> 6;
    if (j < m) {
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
      for (int k = 0; k < m; ++k) {
        const double bk = B[k * TINY_M + j];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += A[(i0 + 16 * r) * TINY_M + k] * bk;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (i0 + 16 * r < m) C[(i0 + 16 * r) * TINY_M + j] = acc[r];
    }
    __syncthreads();
  };
  // (Q X)[i][l] for every (i, l), or X when Q == NULL: each work item is one
  // column l and 8 consecutive rows, so the loads of X[k][l] are coalesced
  // across the lanes and Q[i][k] is the same address for all of them
  auto apply = [&](const double* Q, auto&& sink) {
    const int groups = (m + 7) / 8;
    for (int it = tid; it < groups * n; it += TINY_THREADS) {
      const int rg = it / n, l = it - (it / n) * n;
      const int i0 = rg * 8;
      double acc[8];
      if (Q) {
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r] = 0.0;
        for (int k = 0; k < m; ++k) {
          const double x = X[(size_t)k * n + l];
#pragma unroll
          for (int r = 0; r < 8; ++r) acc[r] += Q[(i0 + r < TINY_M ? i0 + r : 0) * TINY_M + k] * x;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r] = i0 + r < m ? X[(size_t)(i0 + r) * n + l] : 0.0;
      }
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (i0 + r < m) sink(i0 + r, l, acc[r]);
    }
  };

  int g = 0, q = -1;
  gram(buf[g]);
  for (int k = 1; k <= K; ++k) {
    const double a = coef[3 * (k - 1)], b = coef[3 * (k - 1) + 1], c = coef[3 * (k - 1) + 2];
    const int p = tiny_free(g, q, -1);
    const int t = tiny_free(g, q, p);
    mm(buf[t], buf[g], buf[g]);                        // G G
    for (int e = tid; e < m * m; e += TINY_THREADS) {  // P = a I + b G + c G G
      const int i = e / m, j = e - (e / m) * m;
      const int o = i * TINY_M + j;
      buf[p][o] = (i == j ? a : 0.0) + b * buf[g][o] + c * buf[t][o];
    }
    __syncthreads();
    if (q < 0) {
      q = p;                                           // Q = P at a segment's first iteration
    } else {
      mm(buf[t], buf[p], buf[q]);                      // Q <- P Q
      q = t;
    }
    if (k == K) break;
    if ((restarts >> (k - 1)) & 1ull) {                // X <- Q X, G <- X X^T, Q <- I
      apply(buf[q], [&](int i, int l, double v) { X2[(size_t)i * n + l] = v; });
      __syncthreads();
      double* tmp = X;
      X = X2;
      X2 = tmp;
      gram(buf[g]);
      q = -1;
    } else {                                           // G <- P (G P)
      const int f = tiny_free(g, p, q);
      mm(buf[f], buf[g], buf[p]);
      mm(buf[g], buf[p], buf[f]);
    }
  }
  // out[rows of S] = (Q X), transposed back when the block is tall
  apply(q < 0 ? nullptr : buf[q], [&](int i, int l, double v) {
    const int sr = d.tall ? l : i, sc = d.tall ? i : l;
    tiny_out(d.out, (size_t)src_row(sr) * d.C + sc, v, fmt);
  });
}

void launch_tiny_gns(const MatDesc* descs, const int* ids, int ntiny, const MatScalars* scalars, const int* idx,
                     const double* coef, int K, unsigned long long restarts, int fmt, hipStream_t s) {
  if (ntiny > 0)
    hipLaunchKernelGGL(k_tiny_gns, dim3(ntiny), dim3(TINY_THREADS), 0, s, descs, ids, scalars, idx, coef, K, restarts,
                       fmt);
}

}  // namespace dion
