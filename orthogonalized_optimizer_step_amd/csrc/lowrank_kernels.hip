// Kernels of the low-rank (Dion / Orth-Dion) step (Orth-Dion explainer,
// technical summary: power iteration, residual buffer, column normalization
// in Dion and QR of the right factor in Orth-Dion).  The rank-r products run
// in k_lr_gemm (lowrank_gemm.hip); what is here is the rest of the step:
//   k_lr_accumulate  B = fl32(M + G) in place (the residual buffer)
//   k_lr_absmax      the largest |value| of B, from k_lr_accumulate's block maxima
//   k_lr_gram_sum    the Gram matrix from its K-chunk partial sums, in fp64
//   k_lr_cholinv     Cholesky factor of an r x r Gram matrix in fp64 and the
//                    inverse of that factor, for CholeskyQR (A = P L^-T)
//   k_lr_colnorm     Dion's column normalization of the right factor
// The second and third raise the max slots that the GEMMs take their fp16
// operand scales from.
#include <hip/hip_runtime.h>

#include "lowrank_internal.h"

namespace dion {

// Accesses to global memory through generic pointers become flat
// instructions, which also count against the LDS wait counter; the
// factorization's and the accumulation's global accesses go through
// global-address-space pointers so that their LDS waits do not wait for them.
#define LR_GLOBAL __attribute__((address_space(1)))
typedef float lr_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t lr_u32x4 __attribute__((ext_vector_type(4)));

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

// the largest value of a block of `nthreads` (at most 1024; every thread
// calls), in thread 0
template <int NTHREADS>
__device__ __forceinline__ float lr_block_max(float mx) {
  __shared__ float red[NTHREADS / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < NTHREADS / 64; ++w) mx = fmaxf(mx, red[w]);
  return mx;
}

// the block's largest value into *slot (non-negative floats order as their bits)
template <int NTHREADS>
__device__ __forceinline__ void lr_raise(unsigned* slot, float mx) {
  mx = lr_block_max<NTHREADS>(mx);
  if (threadIdx.x == 0 && mx > 0.f) atomicMax(slot, __float_as_uint(mx));
}

}  // namespace

// B = fl32(M + G): one correctly rounded addition per element, 8 per thread;
// the block's largest |B| goes to blockmax[block] (k_lr_absmax reduces them:
// atomics to one address per matrix from every block would serialize).
__global__ __launch_bounds__(256) void k_lr_accumulate(const LrDesc* __restrict__ descs, int nmat, int fmt,
                                                       float* __restrict__ blockmax) {
  const int64_t b = blockIdx.x;
  const LrDesc& d = descs[lr_mat_of_block(descs, nmat, b)];
  const int64_t e0 = (b - d.blk0) * LR_BLOCK_ELEMS + (int64_t)threadIdx.x * 8;
  float mx = 0.f;
  if (e0 < d.elems) {
    float LR_GLOBAL* M = (float LR_GLOBAL*)d.M + e0;
    const char LR_GLOBAL* G = (const char LR_GLOBAL*)d.G + e0 * (fmt == 1 ? 4 : 2);
    // 16-byte accesses: M's 8 values as two, G's as one (16-bit) or two (fp32)
    if (e0 + 8 <= d.elems && ((uintptr_t)M & 31) == 0 && ((uintptr_t)G & 15) == 0) {
      const lr_f32x4 m0 = ((const lr_f32x4 LR_GLOBAL*)M)[0], m1 = ((const lr_f32x4 LR_GLOBAL*)M)[1];
      float m[8] = {m0[0], m0[1], m0[2], m0[3], m1[0], m1[1], m1[2], m1[3]};
      float g[8];
      if (fmt == 1) {
        const lr_f32x4 g0 = ((const lr_f32x4 LR_GLOBAL*)G)[0], g1 = ((const lr_f32x4 LR_GLOBAL*)G)[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          g[i] = g0[i];
          g[4 + i] = g1[i];
        }
      } else {
        const lr_u32x4 u = *(const lr_u32x4 LR_GLOBAL*)G;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t h = (u[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
          g[i] = fmt == 0 ? __uint_as_float(h << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)h);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        m[i] = __fadd_rn(m[i], g[i]);
        mx = fmaxf(mx, fabsf(m[i]));
      }
      ((lr_f32x4 LR_GLOBAL*)M)[0] = lr_f32x4{m[0], m[1], m[2], m[3]};
      ((lr_f32x4 LR_GLOBAL*)M)[1] = lr_f32x4{m[4], m[5], m[6], m[7]};
    } else {
      for (int i = 0; i < 8 && e0 + i < d.elems; ++i) {
        M[i] = __fadd_rn(M[i], lr_in(d.G, e0 + i, fmt));
        mx = fmaxf(mx, fabsf(M[i]));
      }
    }
  }
  mx = lr_block_max<256>(mx);
  if (threadIdx.x == 0) blockmax[b] = mx;
}

// Grid (LR_ABSMAX_SPLIT, matrices): block x of matrix i reduces its share of
// the matrix's block maxima from k_lr_accumulate into the LS_B slot.
__global__ __launch_bounds__(256) void k_lr_absmax(const LrDesc* __restrict__ descs,
                                                   const float* __restrict__ blockmax) {
  const LrDesc& d = descs[blockIdx.y];
  const int parts = gridDim.x, part = blockIdx.x, tid = threadIdx.x;
  const int64_t nb = (d.elems + LR_BLOCK_ELEMS - 1) / LR_BLOCK_ELEMS;
  float mb = 0.f;
  for (int64_t e = (int64_t)part * 256 + tid; e < nb; e += (int64_t)parts * 256) mb = fmaxf(mb, blockmax[d.blk0 + e]);
  lr_raise<256>(d.amax + LS_B, mb);
}

// A64 = S in fp64: on and below the diagonal the sum of the partial Grams of
// the K chunks (parts_R or parts_C of them), added in order; zero above it.
// The input of both factorization kernels.  Grid (LR_SUM_SPLIT, matrices),
// each thread a few entries (four partials' loads in flight at a time).
__global__ __launch_bounds__(256) void k_lr_gram_sum(const LrDesc* __restrict__ descs, int rows_are_R) {
  const LrDesc& d = descs[blockIdx.y];
  const int parts = rows_are_R ? d.parts_R : d.parts_C;
  const int r = d.r;
  const size_t rr = (size_t)r * r;
  const float LR_GLOBAL* S = (const float LR_GLOBAL*)d.S;
  double LR_GLOBAL* A = (double LR_GLOBAL*)d.A64;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < rr; e += (size_t)gridDim.x * 256) {
    const size_t i = e / r, j = e - i * r;
    double v = 0.0;
    if (j <= i) {
      int p = 0;
      for (; p + 4 <= parts; p += 4) {
        const float a0 = S[p * rr + e], a1 = S[(p + 1) * rr + e], a2 = S[(p + 2) * rr + e], a3 = S[(p + 3) * rr + e];
        v += (double)a0;
        v += (double)a1;
        v += (double)a2;
        v += (double)a3;
      }
      for (; p < parts; ++p) v += (double)S[p * rr + e];
    }
    A[e] = v;
  }
}

// One block per matrix.  From the Gram S = F^T F (r x r, in A64 as
// k_lr_gram_sum leaves it: fp64, lower triangle, zero above) of the factor
// F being orthogonalized, factored in place: the lower Cholesky factor L of S, in
// fp64, then Linv = L^-1 (fp32, lower; zero above the diagonal), so that
// F L^-T has orthonormal columns (CholeskyQR; the triangular factor L^T has
// a positive diagonal).  Left-looking: column j takes the dot products of
// rows i >= j with row j over the finished columns k < j, then is scaled by
// the pivot.  A pivot at most 1e-14 times the largest diagonal entry of S
// counts as zero (the factor is rank-deficient, outside the method's
// contract): its column of L^-1 and of the result is zero, which keeps every
// value finite.  The inverse is column-wise forward substitution, one column
// per thread, X = L^-1 kept transposed in the upper triangle of the scratch.
__global__ __launch_bounds__(256) void k_lr_cholinv(const LrDesc* __restrict__ descs, float shift, int amax_slot) {
  const LrDesc& d = descs[blockIdx.x];
  const int r = d.r;
  if (r <= LR_REG_RMAX) return;   // k_lr_cholinv_reg
  const int tid = threadIdx.x;
  double* A = d.A64;
  __shared__ double rowj[512];
  __shared__ double diag[512];
  __shared__ double red[256];

  double mx = 0.0;
  for (int i = tid; i < r; i += 256) mx = fmax(mx, A[(size_t)i * r + i]);   // A = S (k_lr_gram_sum)
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
  float mxl = 0.f;
  for (int e = tid; e < r * r; e += 256) {
    const int i = e / r, c = e - (e / r) * r;
    const float x = i >= c ? (float)A[(size_t)c * r + i] : 0.f;
    d.Linv[e] = x;
    mxl = fmaxf(mxl, fabsf(x));
  }
  lr_raise<256>(d.amax + amax_slot, mxl);
}

// The same factorization for r <= 256 with the lower triangle held in
// registers: 1024 threads as a 32 x 32 grid, thread (ty, tx) owning the
// entries (ty + 32 a, tx + 32 b), a >= b, of the 8 x 8 block-cyclic layout (36
// fp64 registers; an entry's row and column follow from its slot, so nothing
// else is stored).  Both are right-looking eliminations with the pivot
// column (and, for the inverse, the finished row) broadcast through LDS:
//   Cholesky, step k: L[k][k] = sqrt(A[k][k]); L[i][k] = A[i][k] / L[k][k];
//     A[i][c] -= L[i][k] L[c][k] for k < c <= i;
//   inverse of L X = I, step k: row k of X divided by L[k][k], then
//     X[i][c] -= L[i][k] X[k][c] for i > k, c <= k.
// They run interleaved, step k of both at once: the inverse's step k needs
// only column k of L, just broadcast, and the registers that held it take
// column k of X.  (A first form stored L to fp64 scratch and reloaded one
// column per inverse step, each step waiting on a global load.)
constexpr int LR_REG_THREADS = 1024;
constexpr int LR_GRID = 32;
constexpr int LR_NB = LR_REG_RMAX / LR_GRID;
constexpr int LR_SLOTS = LR_NB * (LR_NB + 1) / 2;
static_assert(LR_GRID * LR_GRID == LR_REG_THREADS, "thread grid");

__global__ __launch_bounds__(1024) void k_lr_cholinv_reg(const LrDesc* __restrict__ descs, float shift,
                                                          int amax_slot) {
  const LrDesc& d = descs[blockIdx.x];
  const int r = d.r;
  if (r > LR_REG_RMAX) return;    // k_lr_cholinv
  const int tid = threadIdx.x;
  const int ty = tid / LR_GRID, tx = tid % LR_GRID;
  __shared__ double u[LR_REG_RMAX];
  __shared__ double red[LR_REG_THREADS / 64];
  __shared__ double s_piv;
  double v[LR_SLOTS];
  // slot of (a, b), a >= b: a (a + 1) / 2 + b
#define LR_FOR_SLOTS(BODY) LR_FOR_SLOTS_IF(true, BODY)
  // only the blocks (a, b) for which USE holds (a condition uniform over the
  // block, so that the others are skipped by a scalar branch)
#define LR_FOR_SLOTS_IF(USE, BODY)                                    \
  _Pragma("unroll") for (int a = 0; a < LR_NB; ++a)                   \
  _Pragma("unroll") for (int b = 0; b <= a; ++b) {                    \
    if (!(USE)) continue;                                             \
    const int sl = a * (a + 1) / 2 + b;                               \
    const int i = ty + LR_GRID * a, c = tx + LR_GRID * b;             \
    const bool own = i < r && (a > b || ty >= tx);                    \
    (void)sl; (void)own;                                              \
    BODY                                                              \
  }
  // S from k_lr_gram_sum; every lane loads (entry 0 for the slots it does
  // not own), so that no load is divergent and all 36 are in flight at once
  const double LR_GLOBAL* S = (const double LR_GLOBAL*)d.A64;
  LR_FOR_SLOTS({
    const double x = S[own ? i * r + c : 0];   // 32-bit offsets from one base
    v[sl] = own ? x : 0.0;
  })
  double mx = 0.0;
  LR_FOR_SLOTS({ if (own && i == c) mx = fmax(mx, v[sl]); })
  for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  double big = 0.0;
  for (int w = 0; w < LR_REG_THREADS / 64; ++w) big = fmax(big, red[w]);
  const double tiny = 1e-14 * big;
  if (shift > 0.f) LR_FOR_SLOTS({ if (own && i == c) v[sl] += (double)shift * big; })

  // Step k finishes column k of L and, with it, row k of X = L^-1: once
  // column k of L is broadcast its slots hold column k of X (zero below the
  // diagonal before this step's update), and the slots of columns c <= k
  // hold X from then on.  One LDS vector u carries both broadcasts, u[c] =
  // X[k][c] for c <= k and L[c][k] for c > k, so that for every row i > k
  // (whose multiplier L[i][k] is u[i]) both updates read
  //   v[i][c] -= u[i] u[c]:
  // the Cholesky trailing update for c > k, the elimination of X for c <= k.
  for (int k = 0; k < r; ++k) {
    const int kb = k / LR_GRID;   // the block row and column of k
    LR_FOR_SLOTS_IF(a == kb && b == kb, { if (own && i == k && c == k) s_piv = v[sl]; })
    __syncthreads();
    const double piv = s_piv;
    const double dk = piv > tiny ? sqrt(piv) : 0.0;
    const double inv = dk > 0.0 ? 1.0 / dk : 0.0;
    LR_FOR_SLOTS_IF(a == kb || b == kb, {
      if (own && c == k) {   // column k of L out to LDS; X[k][k] = 1 / L[k][k], X[i][k] = 0 (i > k)
        u[i] = i == k ? inv : v[sl] * inv;
        v[sl] = i == k ? inv : 0.0;
      } else if (own && i == k && c < k) {   // the rest of row k of X
        v[sl] *= inv;
        u[c] = v[sl];
      }
    })
    __syncthreads();
    LR_FOR_SLOTS_IF(a >= kb, { if (own && i > k) v[sl] -= u[i] * u[c]; })   // rows above block kb are done
  }
  float LR_GLOBAL* Linv = (float LR_GLOBAL*)d.Linv;
  for (int e = tid; e < r * r; e += LR_REG_THREADS) {
    const int i = e / r, c = e - (e / r) * r;
    if (c > i) Linv[e] = 0.f;
  }
  float mxl = 0.f;
  LR_FOR_SLOTS({
    if (own) {
      const float x = (float)v[sl];
      Linv[(size_t)i * r + c] = x;
      mxl = fmaxf(mxl, fabsf(x));
    }
  })
  lr_raise<LR_REG_THREADS>(d.amax + amax_slot, mxl);
#undef LR_FOR_SLOTS
#undef LR_FOR_SLOTS_IF
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

void launch_lr_accumulate(const LrDesc* d, int nmat, int64_t blocks, int grad_fmt, float* blockmax, hipStream_t s) {
  if (blocks > 0)
    hipLaunchKernelGGL(k_lr_accumulate, dim3((unsigned)blocks), dim3(256), 0, s, d, nmat, grad_fmt, blockmax);
}
void launch_lr_absmax(const LrDesc* d, int nmat, const float* blockmax, hipStream_t s) {
  if (nmat > 0) hipLaunchKernelGGL(k_lr_absmax, dim3(LR_ABSMAX_SPLIT, nmat), dim3(256), 0, s, d, blockmax);
}
void launch_lr_cholinv(const LrDesc* d, int nmat, bool any_small, bool any_large, bool rows_are_R, float shift,
                       int amax_slot, hipStream_t s) {
  if (nmat <= 0) return;
  hipLaunchKernelGGL(k_lr_gram_sum, dim3(LR_SUM_SPLIT, nmat), dim3(256), 0, s, d, rows_are_R ? 1 : 0);
  if (any_small) hipLaunchKernelGGL(k_lr_cholinv_reg, dim3(nmat), dim3(LR_REG_THREADS), 0, s, d, shift, amax_slot);
  if (any_large) hipLaunchKernelGGL(k_lr_cholinv, dim3(nmat), dim3(256), 0, s, d, shift, amax_slot);
}
void launch_lr_colnorm(const LrDesc* d, int nmat, hipStream_t s) {
  if (nmat > 0) hipLaunchKernelGGL(k_lr_colnorm, dim3(nmat), dim3(256), 0, s, d);
}

}  // namespace dion
