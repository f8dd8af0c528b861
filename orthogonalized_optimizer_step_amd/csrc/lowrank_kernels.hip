// Kernels of the low-rank (Dion / Orth-Dion) step (Orth-Dion explainer,
// technical summary: power iteration, residual buffer, column normalization
// in Dion and QR of the right factor in Orth-Dion).  The rank-r products run
// as batched GEMMs in rocBLAS; what is here is the rest of the step:
//   k_lr_accumulate  B = fl32(M + G) in place (the residual buffer)
//   k_lr_cholinv     Cholesky factor of an r x r Gram matrix in fp64 and the
//                    inverse of that factor, for CholeskyQR (A = P L^-T)
//   k_lr_colnorm     Dion's column normalization of the right factor
//   k_lr_cast        the fp32 update to bf16 or fp16, round to nearest even
#include <hip/hip_runtime.h>

#include "lowrank_internal.h"

namespace dion {

namespace {

__device__ __forceinline__ int lr_mat_of_block(const LrDesc* d, int nmat, int64_t b) {
  int lo = 0, hi = nmat;  // d[lo].blk0 <= b < d[hi].blk0
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (d[mid].blk0 <= b) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ float lr_in(const void* p, int64_t e, int fmt) {
  if (fmt == 1) return ((const float*)p)[e];
  const uint16_t u = ((const uint16_t*)p)[e];
  if (fmt == 0) return __uint_as_float((uint32_t)u << 16);
  return (float)__builtin_bit_cast(_Float16, u);
}

__device__ __forceinline__ uint16_t lr_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace

// B = fl32(M + G): one correctly rounded addition per element, 8 per thread.
__global__ __launch_bounds__(256) void k_lr_accumulate(const LrDesc* __restrict__ descs, int nmat, int fmt) {
  const int64_t b = blockIdx.x;
  const LrDesc& d = descs[lr_mat_of_block(descs, nmat, b)];
  const int64_t e0 = (b - d.blk0) * LR_BLOCK_ELEMS + (int64_t)threadIdx.x * 8;
  if (e0 >= d.elems) return;
  float* M = d.M + e0;
  if (e0 + 8 <= d.elems && ((uintptr_t)M & 31) == 0) {
    float4 m0 = *(const float4*)M, m1 = *(const float4*)(M + 4);
    float g[8];
    if (fmt == 1 && ((uintptr_t)((const float*)d.G + e0) & 15) == 0) {
      const float4 g0 = *(const float4*)((const float*)d.G + e0), g1 = *(const float4*)((const float*)d.G + e0 + 4);
      g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w; g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) g[i] = lr_in(d.G, e0 + i, fmt);
    }
    m0.x = __fadd_rn(m0.x, g[0]); m0.y = __fadd_rn(m0.y, g[1]); m0.z = __fadd_rn(m0.z, g[2]); m0.w = __fadd_rn(m0.w, g[3]);
    m1.x = __fadd_rn(m1.x, g[4]); m1.y = __fadd_rn(m1.y, g[5]); m1.z = __fadd_rn(m1.z, g[6]); m1.w = __fadd_rn(m1.w, g[7]);
    *(float4*)M = m0;
    *(float4*)(M + 4) = m1;
  } else {
    for (int i = 0; i < 8 && e0 + i < d.elems; ++i) M[i] = __fadd_rn(M[i], lr_in(d.G, e0 + i, fmt));
  }
}

// The fp32 update D to the output dtype (0 bf16, 2 fp16), 8 elements per thread.
__global__ __launch_bounds__(256) void k_lr_cast(const LrDesc* __restrict__ descs, int nmat, int fmt) {
  const int64_t b = blockIdx.x;
  const LrDesc& d = descs[lr_mat_of_block(descs, nmat, b)];
  const int64_t e0 = (b - d.blk0) * LR_BLOCK_ELEMS + (int64_t)threadIdx.x * 8;
  if (e0 >= d.elems) return;
  const float* D = d.D + e0;
  uint16_t* o = (uint16_t*)d.out + e0;
  const int n = e0 + 8 <= d.elems ? 8 : (int)(d.elems - e0);
  float v[8];
  if (n == 8 && ((uintptr_t)D & 15) == 0) {
    *(float4*)&v[0] = *(const float4*)D;
    *(float4*)&v[4] = *(const float4*)(D + 4);
  } else {
    for (int i = 0; i < n; ++i) v[i] = D[i];
  }
  uint16_t h[8];
  for (int i = 0; i < n; ++i)
    h[i] = fmt == 0 ? lr_bf16_rne(v[i]) : __builtin_bit_cast(uint16_t, (_Float16)v[i]);
  if (n == 8 && ((uintptr_t)o & 15) == 0) {
    uint4 pk;
    pk.x = h[0] | ((uint32_t)h[1] << 16);
    pk.y = h[2] | ((uint32_t)h[3] << 16);
    pk.z = h[4] | ((uint32_t)h[5] << 16);
    pk.w = h[6] | ((uint32_t)h[7] << 16);
    *(uint4*)o = pk;
  } else {
    for (int i = 0; i < n; ++i) o[i] = h[i];
  }
}

// One block per matrix.  From the Gram S = F^T F (r x r, fp32, symmetric) of
// the factor F being orthogonalized: the lower Cholesky factor L of S, in
// fp64, then Linv = L^-1 (fp32, lower; zero above the diagonal), so that
// F L^-T has orthonormal columns (CholeskyQR; the triangular factor L^T has
// a positive diagonal).  Left-looking: column j takes the dot products of
// rows i >= j with row j over the finished columns k < j, then is scaled by
// the pivot.  A pivot at most 1e-14 times the largest diagonal entry of S
// counts as zero (the factor is rank-deficient, outside the method's
// contract): its column of L^-1 and of the result is zero, which keeps every
// value finite.  The inverse is column-wise forward substitution, one column
// per thread, X = L^-1 kept transposed in the upper triangle of the scratch.
__global__ __launch_bounds__(256) void k_lr_cholinv(const LrDesc* __restrict__ descs, float shift) {
  const LrDesc& d = descs[blockIdx.x];
  const int r = d.r;
  if (r <= LR_REG_RMAX) return;   // k_lr_cholinv_reg
  const int tid = threadIdx.x;
  double* A = d.A64;
  __shared__ double rowj[512];
  __shared__ double diag[512];
  __shared__ double red[256];

  double mx = 0.0;
  for (int e = tid; e < r * r; e += 256) {
    const int i = e / r, j = e - (e / r) * r;
    const double v = j <= i ? (double)d.S[e] : 0.0;
    A[e] = v;
    if (i == j) mx = fmax(mx, v);
  }
  red[tid] = mx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] = fmax(red[tid], red[tid + s]);
    __syncthreads();
  }
  const double tiny = 1e-14 * red[0];
  // shifted pass: S + shift * max_i S_ii * I (every thread has read red[0]
  // before the first barrier of the loop below, which orders these writes)
  if (shift > 0.f)
    for (int i = tid; i < r; i += 256) A[(size_t)i * r + i] += (double)shift * red[0];

  for (int j = 0; j < r; ++j) {
    for (int k = tid; k < j; k += 256) rowj[k] = A[(size_t)j * r + k];
    __syncthreads();
    for (int i = j + tid; i < r; i += 256) {
      const double* Ai = A + (size_t)i * r;
      double s = Ai[j];
      for (int k = 0; k < j; ++k) s -= Ai[k] * rowj[k];
      A[(size_t)i * r + j] = s;
    }
    __syncthreads();
    const double dsq = A[(size_t)j * r + j];
    const double dj = dsq > tiny ? sqrt(dsq) : 0.0;
    for (int i = j + 1 + tid; i < r; i += 256) {
      const double v = A[(size_t)i * r + j];
      A[(size_t)i * r + j] = dj > 0.0 ? v / dj : 0.0;
    }
    if (tid == 0) diag[j] = dj;
    __syncthreads();
  }

  // X = L^-1: X[c][c] = 1 / L[c][c]; X[i][c] = -(sum_{c<=k<i} L[i][k] X[k][c]) / L[i][i].
  // L[i][k] (k < i) is A[i][k]; X[k][c] (k >= c) is stored at A[c][k].
  for (int c = tid; c < r; c += 256) {
    double* Xc = A + (size_t)c * r;
    Xc[c] = diag[c] > 0.0 ? 1.0 / diag[c] : 0.0;
    for (int i = c + 1; i < r; ++i) {
      const double* Li = A + (size_t)i * r;
      double s = 0.0;
      for (int k = c; k < i; ++k) s += Li[k] * Xc[k];
      Xc[i] = diag[i] > 0.0 ? -s / diag[i] : 0.0;
    }
  }
  __syncthreads();
  for (int e = tid; e < r * r; e += 256) {
    const int i = e / r, c = e - (e / r) * r;
    d.Linv[e] = i >= c ? (float)A[(size_t)c * r + i] : 0.f;
  }
}

// The same factorization for r <= 256 with the lower triangle held in
// registers: 1024 threads as a 32 x 32 grid, thread (ty, tx) owning the
// entries (ty + 32 a, tx + 32 b), a >= b, of the 8 x 8 block-cyclic layout (36
// fp64 registers; an entry's row and column follow from its slot, so nothing
// else is stored).  Both steps are right-looking eliminations with the pivot
// column (and, for the inverse, the finished row) broadcast through LDS:
//   Cholesky, step k: L[k][k] = sqrt(A[k][k]); L[i][k] = A[i][k] / L[k][k];
//     A[i][c] -= L[i][k] L[c][k] for k < c <= i;
//   inverse of L X = I, step k: row k of X divided by L[k][k], then
//     X[i][c] -= L[i][k] X[k][c] for i > k, c <= k.
// L leaves the registers for the fp64 scratch (column-major, so that a
// column is one contiguous read) before the inverse reuses them.
constexpr int LR_REG_THREADS = 1024;
constexpr int LR_GRID = 32;
constexpr int LR_NB = LR_REG_RMAX / LR_GRID;
constexpr int LR_SLOTS = LR_NB * (LR_NB + 1) / 2;
static_assert(LR_GRID * LR_GRID == LR_REG_THREADS, "thread grid");

__global__ __launch_bounds__(1024) void k_lr_cholinv_reg(const LrDesc* __restrict__ descs, float shift) {
  const LrDesc& d = descs[blockIdx.x];
  const int r = d.r;
  if (r > LR_REG_RMAX) return;    // k_lr_cholinv
  const int tid = threadIdx.x;
  const int ty = tid / LR_GRID, tx = tid % LR_GRID;
  __shared__ double col[LR_REG_RMAX];
  __shared__ double rowx[LR_REG_RMAX];
  __shared__ double diag[LR_REG_RMAX];
  __shared__ double red[LR_REG_THREADS / 64];
  __shared__ double s_piv;
  double v[LR_SLOTS];
  // slot of (a, b), a >= b: a (a + 1) / 2 + b
#define LR_FOR_SLOTS(BODY)                                            \
  _Pragma("unroll") for (int a = 0; a < LR_NB; ++a)                   \
  _Pragma("unroll") for (int b = 0; b <= a; ++b) {                    \
    const int sl = a * (a + 1) / 2 + b;                               \
    const int i = ty + LR_GRID * a, c = tx + LR_GRID * b;             \
    const bool own = i < r && (a > b || ty >= tx);                    \
    (void)sl; (void)own;                                              \
    BODY                                                              \
  }
  double mx = 0.0;
  LR_FOR_SLOTS({
    v[sl] = own ? (double)d.S[(size_t)i * r + c] : 0.0;
    if (own && i == c) mx = fmax(mx, v[sl]);
  })
  for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  double big = 0.0;
  for (int w = 0; w < LR_REG_THREADS / 64; ++w) big = fmax(big, red[w]);
  const double tiny = 1e-14 * big;
  if (shift > 0.f) LR_FOR_SLOTS({ if (own && i == c) v[sl] += (double)shift * big; })

  for (int k = 0; k < r; ++k) {
    LR_FOR_SLOTS({ if (own && i == k && c == k) s_piv = v[sl]; })
    __syncthreads();
    const double piv = s_piv;
    const double dk = piv > tiny ? sqrt(piv) : 0.0;
    const double inv = dk > 0.0 ? 1.0 / dk : 0.0;
    LR_FOR_SLOTS({
      if (own && c == k) {
        const double x = i == k ? dk : v[sl] * inv;
        v[sl] = x;
        col[i] = x;
      }
    })
    if (tid == 0) diag[k] = dk;
    __syncthreads();
    LR_FOR_SLOTS({ if (own && c > k) v[sl] -= col[i] * col[c]; })
  }
  // L (column-major) to the scratch; X = I in the registers
  double* Lc = d.A64;
  LR_FOR_SLOTS({
    if (own) Lc[(size_t)c * r + i] = v[sl];
    v[sl] = (own && i == c) ? 1.0 : 0.0;
  })
  __syncthreads();
  for (int k = 0; k < r; ++k) {
    for (int i = k + 1 + tid; i < r; i += LR_REG_THREADS) col[i] = Lc[(size_t)k * r + i];
    const double dinv = diag[k] > 0.0 ? 1.0 / diag[k] : 0.0;
    LR_FOR_SLOTS({
      if (own && i == k) {
        v[sl] *= dinv;
        rowx[c] = v[sl];
      }
    })
    __syncthreads();
    LR_FOR_SLOTS({ if (own && i > k && c <= k) v[sl] -= col[i] * rowx[c]; })
    __syncthreads();
  }
  for (int e = tid; e < r * r; e += LR_REG_THREADS) {
    const int i = e / r, c = e - (e / r) * r;
    if (c > i) d.Linv[e] = 0.f;
  }
  LR_FOR_SLOTS({ if (own) d.Linv[(size_t)i * r + c] = (float)v[sl]; })
#undef LR_FOR_SLOTS
}

// One block per matrix: Q[:, j] = W[:, j] / ||W[:, j]|| (fp64 norm), zero
// columns stay zero (Dion's column normalization).
__global__ __launch_bounds__(256) void k_lr_colnorm(const LrDesc* __restrict__ descs) {
  const LrDesc& d = descs[blockIdx.x];
  const int r = d.r, C = d.C;
  for (int j = threadIdx.x; j < r; j += 256) {
    double s = 0.0;
    for (int i = 0; i < C; ++i) {
      const double w = d.W[(size_t)i * r + j];
      s += w * w;
    }
    const double inv = s > 0.0 ? 1.0 / sqrt(s) : 0.0;
    for (int i = 0; i < C; ++i) d.Q[(size_t)i * r + j] = (float)((double)d.W[(size_t)i * r + j] * inv);
  }
}

void launch_lr_accumulate(const LrDesc* d, int nmat, int64_t blocks, int grad_fmt, hipStream_t s) {
  if (blocks > 0) hipLaunchKernelGGL(k_lr_accumulate, dim3((unsigned)blocks), dim3(256), 0, s, d, nmat, grad_fmt);
}
void launch_lr_cast(const LrDesc* d, int nmat, int64_t blocks, int out_fmt, hipStream_t s) {
  if (blocks > 0) hipLaunchKernelGGL(k_lr_cast, dim3((unsigned)blocks), dim3(256), 0, s, d, nmat, out_fmt);
}
void launch_lr_cholinv(const LrDesc* d, int nmat, bool any_small, bool any_large, float shift, hipStream_t s) {
  if (nmat > 0 && any_small) hipLaunchKernelGGL(k_lr_cholinv_reg, dim3(nmat), dim3(LR_REG_THREADS), 0, s, d, shift);
  if (nmat > 0 && any_large) hipLaunchKernelGGL(k_lr_cholinv, dim3(nmat), dim3(256), 0, s, d, shift);
}
void launch_lr_colnorm(const LrDesc* d, int nmat, hipStream_t s) {
  if (nmat > 0) hipLaunchKernelGGL(k_lr_colnorm, dim3(nmat), dim3(256), 0, s, d);
}

}  // namespace dion
