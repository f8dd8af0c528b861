// Gram Newton-Schulz for small matrices in one launch (Dion3 summary,
// 方法 / 核心模块, "Gram Newton-Schulz" bullet: G = X X^T, then per iteration
// P = aI + bG + cG^2, Q <- P Q, and G <- P G P or, at a restart, X <- Q X,
// G <- X X^T, Q <- I; out = Q X).
//
// For matrices whose Gram side m is at most 64 (and long side at most 1024,
// or any long side when m is at most 16) the GEMM phases would be some twenty
// launches of a tile or three each, so a call of only such matrices is bound
// by launch latency, and beside larger ones they would take 256-row tiles for
// a few rows, whose fp16 rounding a Gram side of a few rows cannot average
// out.  Here one workgroup per matrix
// runs the whole iteration in fp64: the m x m matrices G, P, Q and a temporary
// live in LDS (four 64 x 64 fp64 buffers, rows padded to 65 so that a column
// of 16 rows spreads over the banks, 133 KB, plus a 16 KB staging chunk for
// the Gram), the iterate X (m x n, fp64) in two workspace buffers that
// alternate at restarts.  The m x m products and the Gram run on the matrix
// cores (v_mfma_f64_16x16x4_f64): each of the 16 waves owns one 16 x 16 tile
// of the 64 x 64 result.  Entries beyond m stay zero in every buffer, so the
// products can run over whole tiles.
#include <hip/hip_runtime.h>

#include "dion_internal.h"

namespace dion {

constexpr int TINY_M = 64;
constexpr int TINY_LD = TINY_M + 1;   // row stride of the LDS matrices
constexpr int TINY_THREADS = 1024;
typedef double tiny_d4 __attribute__((ext_vector_type(4)));
#define TINY_GLOBAL __attribute__((address_space(1)))

namespace {

__device__ __forceinline__ double tiny_in(const void* p, size_t e, int fmt) {
  if (fmt == 1) return (double)((const float*)p)[e];
  const uint16_t u = ((const uint16_t*)p)[e];
  if (fmt == 0) return (double)__uint_as_float((uint32_t)u << 16);
  return (double)(float)__builtin_bit_cast(_Float16, u);
}

// the result's element (rounded to fp32 first), or with `update` the weight
// update of the row-subset step: W <- fl32(fl32(W * keep) - fl32(alpha * u)),
// u = the fp32 result, then rounded to W's dtype
__device__ __forceinline__ void tiny_out(void* p, size_t e, double v, int fmt, int update, float keep,
                                         float alpha) {
  float f = (float)v;
  if (update) {
    const float cur = fmt == 1 ? ((const float*)p)[e] : __uint_as_float((uint32_t)((const uint16_t*)p)[e] << 16);
    f = __fsub_rn(__fmul_rn(cur, keep), __fmul_rn(alpha, f));
  }
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
// restarts: bit k-1 set = restart after iteration k; in_fmt, out_fmt: element
// formats of M and out (0 bf16, 1 fp32, 2 fp16); update: out is the weight W
// of the row-subset step's fused update (bf16 or fp32), with the decay factor
// keep and the matrix's alpha.
__global__ __launch_bounds__(TINY_THREADS) void k_tiny_gns(const MatDesc* __restrict__ descs,
                                                           const int* __restrict__ ids,
                                                           const MatScalars* __restrict__ scalars,
                                                           const int* __restrict__ idx,
                                                           const double* __restrict__ coef, int K,
                                                           unsigned long long restarts, int in_fmt,
                                                           int out_fmt, int update, float keep) {
  const int mi = ids[blockIdx.x];
  const MatDesc& d = descs[mi];
  const int m = d.m, n = d.n;
  const int tid = threadIdx.x;
  const double nu2 = scalars[mi].nu2;                // ||S||_F^2 from the selection
  const double s = nu2 > 0.0 ? 1.0 / sqrt(nu2) : 0.0;
  __shared__ double buf[4][TINY_M * TINY_LD];         // row-major, ld TINY_LD
  double TINY_GLOBAL* X = (double TINY_GLOBAL*)d.buf[SLOT_X];     // m x n, ld n
  double TINY_GLOBAL* X2 = (double TINY_GLOBAL*)d.buf[SLOT_XT0];
  for (int e = tid; e < 4 * TINY_M * TINY_LD; e += TINY_THREADS) (&buf[0][0])[e] = 0.0;
  auto src_row = [&](int j) { return idx ? idx[d.sel0 + j] : j; };

  // X = S / nu, oriented so that m <= n (S^T when the block is tall)
  for (int e = tid; e < m * n; e += TINY_THREADS) {
    const int i = e / n, l = e - (e / n) * n;
    const int sr = d.tall ? l : i, sc = d.tall ? i : l;
    X[e] = tiny_in(d.M, (size_t)src_row(sr) * d.C + sc, in_fmt) * s;
  }
  __syncthreads();

  // The MFMA tiles: wave w owns rows 16 (w / 4) .. + 15 and columns 16 (w %
  // 4) .. + 15 of a 64 x 64 result.  v_mfma_f64_16x16x4_f64 takes lane l's
  // A[l % 16][l / 16] and B[l / 16][l % 16] and accumulates D[l / 16 +
  // 4 v][l % 16] in its element v (rows interleaved by four; checked on the
  // device against a host product).  Tiles wholly beyond m are zero.
  const int lane = tid & 63, wave = tid >> 6;
  const int ti = wave >> 2, tj = wave & 3;
  const bool live = ti * 16 < m && tj * 16 < m;
  auto tile_store = [&](double* C, const tiny_d4& acc) {
#pragma unroll
    for (int v = 0; v < 4; ++v) C[(ti * 16 + (lane >> 4) + 4 * v) * TINY_LD + tj * 16 + (lane & 15)] = acc[v];
  };
  // G = X X^T from 32-column chunks of X staged transposed in LDS (xc[k][row]);
  // G[i][j] and G[j][i] take the same products in the same order
  __shared__ double xc[32 * TINY_M];
  auto gram = [&](double* G) {
    tiny_d4 acc = {0.0, 0.0, 0.0, 0.0};
    for (int l0 = 0; l0 < n; l0 += 32) {
      for (int e = tid; e < 32 * TINY_M; e += TINY_THREADS) {
        const int row = e >> 5, k = e & 31;
        xc[k * TINY_M + row] = (row < m && l0 + k < n) ? X[(size_t)row * n + l0 + k] : 0.0;
      }
      __syncthreads();
      if (live) {
#pragma unroll
        for (int k0 = 0; k0 < 32; k0 += 4) {
          const int k = k0 + (lane >> 4);
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xc[k * TINY_M + ti * 16 + (lane & 15)],
                                                     xc[k * TINY_M + tj * 16 + (lane & 15)], acc, 0, 0, 0);
        }
      }
      __syncthreads();
    }
    tile_store(G, acc);
    __syncthreads();
  };
  // C = A B (m x m, zero beyond m); C is neither A nor B
  const int kmax = (m + 3) & ~3;
  auto mm = [&](double* C, const double* A, const double* B) {
    tiny_d4 acc = {0.0, 0.0, 0.0, 0.0};
    if (live) {
      for (int k0 = 0; k0 < kmax; k0 += 4) {
        const int k = k0 + (lane >> 4);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(A[(ti * 16 + (lane & 15)) * TINY_LD + k],
                                                   B[k * TINY_LD + tj * 16 + (lane & 15)], acc, 0, 0, 0);
      }
    }
    tile_store(C, acc);
    __syncthreads();
  };
  // P = a I + b G + c G G, the polynomial formed from G G's tiles as they
  // leave the matrix cores (zero beyond m)
  auto mm_poly = [&](double* P, const double* G, double a, double b, double c) {
    tiny_d4 acc = {0.0, 0.0, 0.0, 0.0};
    if (live) {
      for (int k0 = 0; k0 < kmax; k0 += 4) {
        const int k = k0 + (lane >> 4);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(G[(ti * 16 + (lane & 15)) * TINY_LD + k],
                                                   G[k * TINY_LD + tj * 16 + (lane & 15)], acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = ti * 16 + (lane >> 4) + 4 * v, j = tj * 16 + (lane & 15);
      const int o = i * TINY_LD + j;
      P[o] = (i < m && j < m) ? (i == j ? a : 0.0) + b * G[o] + c * acc[v] : 0.0;
    }
    __syncthreads();
  };
  // (Q X)[i][l] for every (i, l), or X when Q == NULL: each wave takes 16 x 16
  // output tiles in turn, the products on the matrix cores with X's values
  // loaded straight from global memory (lane l: row k0 + l / 16, column l % 16)
  auto apply = [&](const double* Q, auto&& sink) {
    const int tiles_l = (n + 15) / 16, tiles = ((m + 15) / 16) * tiles_l;
    for (int tt = wave; tt < tiles; tt += TINY_THREADS / 64) {
      const int ai = tt / tiles_l, al = tt - (tt / tiles_l) * tiles_l;
      const int col = al * 16 + (lane & 15);
      tiny_d4 acc = {0.0, 0.0, 0.0, 0.0};
      if (Q) {
#pragma unroll 4
        for (int k0 = 0; k0 < kmax; k0 += 4) {
          const int k = k0 + (lane >> 4);
          const double x = (k < m && col < n) ? X[(size_t)k * n + col] : 0.0;
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(Q[(ai * 16 + (lane & 15)) * TINY_LD + k], x, acc, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int i = ai * 16 + (lane >> 4) + 4 * v;
          acc[v] = (i < m && col < n) ? X[(size_t)i * n + col] : 0.0;
        }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = ai * 16 + (lane >> 4) + 4 * v;
        if (i < m && col < n) sink(i, col, acc[v]);
      }
    }
  };

  int g = 0, q = -1;
  gram(buf[g]);
  for (int k = 1; k <= K; ++k) {
    const double a = coef[3 * (k - 1)], b = coef[3 * (k - 1) + 1], c = coef[3 * (k - 1) + 2];
    const int p = tiny_free(g, q, -1);
    mm_poly(buf[p], buf[g], a, b, c);                  // P = a I + b G + c G G
    if (q < 0) {
      q = p;                                           // Q = P at a segment's first iteration
    } else {
      const int t = tiny_free(g, q, p);
      mm(buf[t], buf[p], buf[q]);                      // Q <- P Q
      q = t;
    }
    if (k == K) break;
    if ((restarts >> (k - 1)) & 1ull) {                // X <- Q X, G <- X X^T, Q <- I
      apply(buf[q], [&](int i, int l, double v) { X2[(size_t)i * n + l] = v; });
      __syncthreads();
      double TINY_GLOBAL* tmp = X;
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
    tiny_out(d.out, (size_t)src_row(sr) * d.C + sc, v, out_fmt, update, keep, d.upd_alpha);
  });
}

void launch_tiny_gns(const MatDesc* descs, const int* ids, int ntiny, const MatScalars* scalars, const int* idx,
                     const double* coef, int K, unsigned long long restarts, int in_fmt, int out_fmt, int update,
                     float keep, hipStream_t s) {
  if (ntiny > 0)
    hipLaunchKernelGGL(k_tiny_gns, dim3(ntiny), dim3(TINY_THREADS), 0, s, descs, ids, scalars, idx, coef, K, restarts,
                       in_fmt, out_fmt, update, keep);
}

}  // namespace dion
