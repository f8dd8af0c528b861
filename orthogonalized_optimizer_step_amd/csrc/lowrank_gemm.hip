// Batched fp32 GEMM of the low-rank (Dion / Orth-Dion) step: every rank-r
// product of the step (Orth-Dion explainer, technical summary: the power
// iteration B Q, the right factor B^T P, the error-feedback update
// B - beta P W^T, the update P Q'^T, and the Gram and apply products of
// CholeskyQR) runs here.
//
//   C = alpha op(A) op(B) + beta C      (row-major fp32, a batch of same-shape
//                                        products given as device pointer arrays)
//
// fp32 accuracy from bf16 matrix cores.  Each fp32 value splits exactly into
// three bf16 terms by truncation: h = x with its low 16 bits cleared, m the
// same of x - h, l = x - h - m (24 significand bits = 8 + 8 + 8; bf16 keeps
// fp32's exponent range, so no operand needs a scale).  A product sums the six
// term products down to relative weight 2^-16 (hh; hm, mh; hl, lh, mm), small
// ones first, in v_mfma_f32_32x32x16_bf16 with fp32 accumulation; the three
// dropped ones weigh 2^-24 and less, the size of fp32's own rounding.
//
// Tiles of 128 x 128 outputs, four waves of 64 x 64 (2 x 2 MFMA blocks).  A
// K-stage of 32 columns is loaded from global memory into registers (16-byte
// loads when the rows allow, zeros outside the matrix) while the previous
// stage is multiplied, then split and stored to LDS as [row][k] bf16 rows of
// four 16-byte chunks per term, the chunk order XOR-swizzled by row so that
// the fragment reads of 32 lanes hit distinct banks.  Operands stored with K
// contiguous are staged row by row; operands stored with M (or N) contiguous
// are staged four K-rows at a time and written as 8-byte column pieces.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace dion {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int LG_TILE = 128;
constexpr int LG_BK = 32;
constexpr int LG_TERM = LG_TILE * LG_BK;   // bf16 elements of one operand term of one stage

// chunk c (8 k values) of row r, swizzled; element offset inside a term
__device__ __forceinline__ int lg_off(int r, int c) { return r * LG_BK + ((c ^ ((r >> 2) & 3)) << 3); }

// x = h + m + l exactly; the three bf16 bit patterns
__device__ __forceinline__ void lg_split(float x, uint32_t& h, uint32_t& m, uint32_t& l) {
  const uint32_t u = __float_as_uint(x);
  h = u >> 16;
  const float r1 = x - __uint_as_float(u & 0xFFFF0000u);
  const uint32_t v = __float_as_uint(r1);
  m = v >> 16;
  const float r2 = r1 - __uint_as_float(v & 0xFFFF0000u);
  l = __float_as_uint(r2) >> 16;   // at most 8 significant bits: exact
}

// A K-stage of one operand: LG_TILE rows (of op(X)'s M or N side) x LG_BK k,
// 16 values per thread.  KC: stored with k contiguous (element (r, k) at
// p[r * ld + k]); otherwise with r contiguous (element (r, k) at p[k * ld + r]).
template <bool KC>
struct LgStage {
  float v[16];
  __device__ __forceinline__ void load(const float* p, int ld, int rows, int ks, int r0, int k0, bool vec) {
    const int t = threadIdx.x;
    if (KC) {   // row r0 + t/2, k0 + (t&1)*16 .. +15
      const int r = r0 + (t >> 1), k = k0 + (t & 1) * 16;
      const float* q = p + (size_t)r * ld + k;
      if (vec && r < rows && k + 16 <= ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *(float4*)&v[4 * i] = ((const float4*)q)[i];
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = (r < rows && k + i < ks) ? q[i] : 0.f;
      }
    } else {    // k0 + (t>>5)*4 + i (i < 4), rows r0 + (t&31)*4 .. +3; v[4 i + j] = (row j, k i)
      const int r = r0 + (t & 31) * 4, k = k0 + (t >> 5) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* q = p + (size_t)(k + i) * ld + r;
        if (vec && k + i < ks && r + 4 <= rows) {
          *(float4*)&v[4 * i] = *(const float4*)q;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) v[4 * i + j] = (k + i < ks && r + j < rows) ? q[j] : 0.f;
        }
      }
    }
  }
  // split and store to the three term arrays at s (bf16 bits as uint16)
  __device__ __forceinline__ void store(uint16_t* s) const {
    const int t = threadIdx.x;
    if (KC) {
      const int r = t >> 1, c0 = (t & 1) * 2;   // chunks c0, c0 + 1
      uint32_t w[3][8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t h0, m0, l0, h1, m1, l1;
        lg_split(v[2 * i], h0, m0, l0);
        lg_split(v[2 * i + 1], h1, m1, l1);
        w[0][i] = h0 | (h1 << 16);
        w[1][i] = m0 | (m1 << 16);
        w[2][i] = l0 | (l1 << 16);
      }
#pragma unroll
      for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          *(uint4*)(s + u * LG_TERM + lg_off(r, c0 + c)) = make_uint4(w[u][4 * c], w[u][4 * c + 1], w[u][4 * c + 2],
                                                                      w[u][4 * c + 3]);
    } else {
      const int r0 = (t & 31) * 4, k = (t >> 5) * 4;   // four rows, k .. k+3
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t h[4], m[4], l[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) lg_split(v[4 * i + j], h[i], m[i], l[i]);
        const int r = r0 + j, o = lg_off(r, k >> 3) + (k & 7);
        *(uint2*)(s + o) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        *(uint2*)(s + LG_TERM + o) = make_uint2(m[0] | (m[1] << 16), m[2] | (m[3] << 16));
        *(uint2*)(s + 2 * LG_TERM + o) = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
      }
    }
  }
};

}  // namespace

// Row-major C (M x N) = alpha op(A) op(B) + beta C for batch entry z =
// blockIdx.z.  A_KC: A is stored M x K (K contiguous, op = N), else K x M
// (op = T).  B_KC: B is stored N x K (op = T), else K x N (op = N).
template <bool A_KC, bool B_KC>
__global__ __launch_bounds__(256) void k_lr_gemm(int M, int N, int K, float alpha, const float* const* __restrict__ As,
                                                 int lda, const float* const* __restrict__ Bs, int ldb, float beta,
                                                 float* const* __restrict__ Cs, int ldc) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[3 * LG_TERM], sB[3 * LG_TERM];
  const int z = blockIdx.z;
  const float* A = As[z];
  const float* B = Bs[z];
  float* C = Cs[z];
  const int m0 = blockIdx.y * LG_TILE, n0 = blockIdx.x * LG_TILE;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bool veca = (lda & 3) == 0 && ((uintptr_t)A & 15) == 0;
  const bool vecb = (ldb & 3) == 0 && ((uintptr_t)B & 15) == 0;

  floatx16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  LgStage<A_KC> ga;
  LgStage<B_KC> gb;
  const int nk = (K + LG_BK - 1) / LG_BK;
  ga.load(A, lda, M, K, m0, 0, veca);
  gb.load(B, ldb, N, K, n0, 0, vecb);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();   // every wave is done with the previous stage
    ga.store(sA);
    gb.store(sB);
    __syncthreads();
    if (kt + 1 < nk) {   // the next stage's loads fly while this one is multiplied
      ga.load(A, lda, M, K, m0, (kt + 1) * LG_BK, veca);
      gb.load(B, ldb, N, K, n0, (kt + 1) * LG_BK, vecb);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int chunk = kk * 2 + (lane >> 5);
      bf16x8 fa[3][2], fb[3][2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int ra = wm * 64 + f * 32 + (lane & 31), rb = wn * 64 + f * 32 + (lane & 31);
#pragma unroll
        for (int u = 0; u < 3; ++u) {
          fa[u][f] = *(const bf16x8*)(sA + u * LG_TERM + lg_off(ra, chunk));
          fb[u][f] = *(const bf16x8*)(sB + u * LG_TERM + lg_off(rb, chunk));
        }
      }
      // term products from the smallest weight: mm, hl, lh (2^-16), hm, mh (2^-8), hh
      constexpr int PA[6] = {1, 0, 2, 0, 1, 0}, PB[6] = {1, 2, 0, 1, 0, 0};
#pragma unroll
      for (int p = 0; p < 6; ++p)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[PA[p]][a], fb[PB[p]][b], acc[a][b], 0, 0, 0);
    }
  }
  // epilogue: lane holds column (lane & 31) of rows (e/4)*8 + (lane/32)*4 + e%4 of each block
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int col = n0 + wn * 64 + b * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * 64 + a * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        if (row < M) {
          float* c = C + (size_t)row * ldc + col;
          const float v = alpha * acc[a][b][e];
          *c = beta != 0.f ? v + beta * *c : v;
        }
      }
    }
}

// Row-major C (m x n) = alpha op(A) op(B) + beta C over `count` pointer
// triples (device arrays): A is m x k (k x m when ta), B is k x n (n x k when
// tb), as the BLAS conventions read in row-major order.
void launch_lr_gemm(bool ta, bool tb, int m, int n, int k, float alpha, const float* const* A, const float* const* B,
                    float beta, float* const* C, int count, hipStream_t s) {
  const int lda = ta ? m : k, ldb = tb ? k : n, ldc = n;
  const dim3 grid((n + LG_TILE - 1) / LG_TILE, (m + LG_TILE - 1) / LG_TILE, count);
  if (!ta && tb)
    hipLaunchKernelGGL((k_lr_gemm<true, true>), grid, dim3(256), 0, s, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc);
  else if (!ta && !tb)
    hipLaunchKernelGGL((k_lr_gemm<true, false>), grid, dim3(256), 0, s, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc);
  else if (ta && !tb)
    hipLaunchKernelGGL((k_lr_gemm<false, false>), grid, dim3(256), 0, s, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc);
  else
    hipLaunchKernelGGL((k_lr_gemm<false, true>), grid, dim3(256), 0, s, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc);
}

}  // namespace dion
