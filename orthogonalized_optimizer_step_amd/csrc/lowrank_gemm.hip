// Batched fp32 GEMM of the low-rank (Dion / Orth-Dion) step: every rank-r
// product of the step (Orth-Dion explainer, technical summary: the power
// iteration B Q, the right factor B^T P, the error-feedback update
// B - beta P W^T, the update P Q'^T, and the Gram and apply products of
// CholeskyQR) runs here.
//
//   C = alpha op(A) op(B) (+ beta C)    (row-major fp32, a batch of same-shape
//                                        products given as device pointer arrays;
//                                        beta C in the split-operand kernel)
//
// fp32 accuracy from 16-bit matrix cores, in one of two operand formats:
//  - F16 (two fp16 terms): each operand is scaled by a power of two s, chosen
//    from its largest |value| (recorded by the operand's producer) so that the
//    largest scaled value lies in [2^13, 2^14), and split as h = fp16(x s),
//    l = fp16(x s - h) (x s - h is exact in fp32): x s = h + l to 22
//    significant bits, or to 2^-24 absolute for the values far below the
//    largest.  A product sums hl, lh and hh in v_mfma_f32_32x32x16_f16 (the
//    dropped ll weighs 2^-22) and is scaled back by 2^-(la + lb), exactly.
//  - BF16x3 (three bf16 terms, no scale): h = x with its low 16 bits cleared,
//    m the same of x - h, l = x - h - m (8 + 8 + 8 significand bits, fp32's
//    exponent range).  A product sums the six term products down to relative
//    weight 2^-16 (mm, hl, lh; hm, mh; hh) in v_mfma_f32_32x32x16_bf16; the
//    dropped ones weigh 2^-24 and less, fp32's own rounding.
// Term products are summed smallest first, with fp32 accumulation.  F16 does
// half the matrix-core work.  Its 22 bits suffice where the result's error
// is not amplified afterwards; the power product B Q, whose result is
// orthogonalized (its error grows with the condition number of B Q), takes
// BF16x3.  In emulation against the fp64 oracle on the randomized low-rank
// draws (ranks up to the full dimension), the worst error is 2.9e-5 with
// BF16x3 everywhere, 7.0e-5 with F16 everywhere and 4.0e-5 with BF16x3 for
// the power product only.
//
// A small F16 operand read by many blocks (P, W and the new Q in the buffer
// update and the update, whose inner dimension is the rank) is split once by
// k_lr_split16 into hi and lo arrays of fp16 rows (K contiguous; rows padded
// to a multiple of 128 and K to a multiple of 32, with zeros), and those two
// products run in k_lr_gemm_dma: its stages go from global memory straight
// into LDS (global_load_lds_dwordx4, each lane's 16 bytes placed where the
// swizzled layout wants them) one stage ahead, with no register staging and
// no split in the kernel.
//
// Tiles of 128 x 128 outputs, four waves of 64 x 64 (2 x 2 MFMA blocks).  A
// K-stage of 32 columns is loaded from global memory into registers (16-byte
// loads for every stage inside the matrix, zeros outside it) while the
// previous stage is multiplied, then split and stored to LDS as [row][k] fp16
// rows of four 16-byte chunks per term, the chunk order XOR-swizzled by row
// so that the fragment reads of 32 lanes hit distinct banks.  Operands stored
// with K contiguous are staged row by row; operands stored with M (or N)
// contiguous are staged four K-rows at a time and written as 8-byte column
// pieces.  The MFMAs take the B operand first, so that the accumulators hold
// C^T and each lane writes four consecutive columns of a row of C at once.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "lowrank_internal.h"

namespace dion {

namespace {

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int LG_TILE = 128;
constexpr int LG_BK = 32;
constexpr int LG_TERM = LG_TILE * LG_BK;   // fp16 elements of one operand term of one stage

// chunk c (8 k values) of row r, swizzled; element offset inside a term
__device__ __forceinline__ int lg_off(int r, int c) { return r * LG_BK + ((c ^ ((r >> 2) & 3)) << 3); }

// log2 of the scale for an operand whose largest |value| has fp32 bits `bits`
// (0 for an all-zero operand); clamped so that 2^l is a normal float
__device__ __forceinline__ int lg_log2_scale(unsigned bits) {
  if (bits == 0u) return 0;
  const int e = (int)(bits >> 23) - 127;   // floor(log2 max) (-127 for a subnormal max)
  return min(max(13 - e, -126), 126);
}

// The terms of x as 16-bit patterns: F16, x s = t[0] + t[1]; BF16x3,
// x = t[0] + t[1] + t[2]
template <bool F16>
__device__ __forceinline__ void lg_split(float x, float s, uint32_t* t) {
  if (F16) {
    const float xs = x * s;
    const _Float16 hh = (_Float16)xs;
    const _Float16 ll = (_Float16)(xs - (float)hh);
    t[0] = __builtin_bit_cast(uint16_t, hh);
    t[1] = __builtin_bit_cast(uint16_t, ll);
  } else {
    const uint32_t u = __float_as_uint(x);
    t[0] = u >> 16;
    const float r1 = x - __uint_as_float(u & 0xFFFF0000u);
    const uint32_t v = __float_as_uint(r1);
    t[1] = v >> 16;
    const float r2 = r1 - __uint_as_float(v & 0xFFFF0000u);
    t[2] = __float_as_uint(r2) >> 16;   // at most 8 significant bits: exact
  }
}

// operand layouts: fp32 with r (the M or N index) contiguous, or with k contiguous
enum { LG_RC = 0, LG_KC = 1 };

// Loads through generic pointers become flat loads, which also count against
// the LDS wait counter: every wait for the fragment reads of a stage would
// then wait for the next stage's loads from memory too.  Operand and result
// accesses therefore go through global-address-space pointers (vmcnt only).
#define LG_GLOBAL __attribute__((address_space(1)))
typedef float lg_float4 __attribute__((ext_vector_type(4)));
typedef uint32_t lg_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t lg_u32x4 __attribute__((ext_vector_type(4)));

// A K-stage of one operand: LG_TILE rows (of op(X)'s M or N side) x LG_BK k,
// 16 values per thread.  KC: stored with k contiguous (element (r, k) at
// p[r * ld + k]); otherwise with r contiguous (element (r, k) at p[k * ld + r]).
template <int MODE, bool F16>
struct LgStage {
  static constexpr bool KC = MODE == LG_KC;
  static constexpr int NT = F16 ? 2 : 3;   // terms
  float v[16];
  // vec: 16-byte aligned rows.  A stage wholly inside the operand (every
  // interior stage) takes 16-byte loads in every lane; the decision is the
  // same for the whole block, so no lane waits on another's loads.
  __device__ __forceinline__ void load(const float* p, int ld, int rows, int ks, int r0, int k0, bool vec) {
    const int t = threadIdx.x;
    const bool whole = vec && r0 + LG_TILE <= rows && k0 + LG_BK <= ks;
    if (KC) {   // row r0 + t/2, k0 + (t&1)*16 .. +15
      const int r = r0 + (t >> 1), k = k0 + (t & 1) * 16;
      const float LG_GLOBAL* q = (const float LG_GLOBAL*)p + (size_t)r * ld + k;
      if (whole) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const lg_float4 x = ((const lg_float4 LG_GLOBAL*)q)[i];
#pragma unroll
          for (int j = 0; j < 4; ++j) v[4 * i + j] = x[j];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = (r < rows && k + i < ks) ? q[i] : 0.f;
      }
    } else {    // k0 + (t>>5)*4 + i (i < 4), rows r0 + (t&31)*4 .. +3; v[4 i + j] = (row j, k i)
      const int r = r0 + (t & 31) * 4, k = k0 + (t >> 5) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float LG_GLOBAL* q = (const float LG_GLOBAL*)p + (size_t)(k + i) * ld + r;
        if (whole) {
          const lg_float4 x = *(const lg_float4 LG_GLOBAL*)q;
#pragma unroll
          for (int j = 0; j < 4; ++j) v[4 * i + j] = x[j];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) v[4 * i + j] = (k + i < ks && r + j < rows) ? q[j] : 0.f;
        }
      }
    }
  }
  // (scale,) split and store to the NT term arrays at s
  __device__ __forceinline__ void store(uint16_t* s, float scale) const {
    const int t = threadIdx.x;
    if (KC) {
      const int r = t >> 1, c0 = (t & 1) * 2;   // chunks c0, c0 + 1
      uint32_t w[NT][8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t a[3], b[3];
        lg_split<F16>(v[2 * i], scale, a);
        lg_split<F16>(v[2 * i + 1], scale, b);
#pragma unroll
        for (int u = 0; u < NT; ++u) w[u][i] = a[u] | (b[u] << 16);
      }
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          *(uint4*)(s + u * LG_TERM + lg_off(r, c0 + c)) = make_uint4(w[u][4 * c], w[u][4 * c + 1], w[u][4 * c + 2],
                                                                      w[u][4 * c + 3]);
    } else {
      const int r0 = (t & 31) * 4, k = (t >> 5) * 4;   // four rows, k .. k+3
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t w[4][3];
#pragma unroll
        for (int i = 0; i < 4; ++i) lg_split<F16>(v[4 * i + j], scale, w[i]);
        const int r = r0 + j, o = lg_off(r, k >> 3) + (k & 7);
#pragma unroll
        for (int u = 0; u < NT; ++u)
          *(uint2*)(s + u * LG_TERM + o) = make_uint2(w[0][u] | (w[1][u] << 16), w[2][u] | (w[3][u] << 16));
      }
    }
  }
};

// The 16-bit gradient G (bf16, gfmt 0, or fp16, gfmt 2) of the residual
// buffer B = fl32(M + G), loaded beside a stage of M in LgStage's element
// order, so that the products that read B take M and G instead of a stored B
// (same rounding: one fl32 addition per element).
template <int MODE>
struct LgGrad {
  static constexpr bool KC = MODE == LG_KC;
  uint32_t w[8];   // two values per word, element i in half i & 1 of word i / 2
  __device__ __forceinline__ void load(const uint16_t* g, int ld, int rows, int ks, int r0, int k0, bool vec) {
    const int t = threadIdx.x;
    const bool whole = vec && r0 + LG_TILE <= rows && k0 + LG_BK <= ks;
    if (KC) {   // row r0 + t/2, k0 + (t&1)*16 .. +15 (16-byte aligned rows: ld a multiple of 8)
      const int r = r0 + (t >> 1), k = k0 + (t & 1) * 16;
      const uint16_t LG_GLOBAL* q = (const uint16_t LG_GLOBAL*)g + (size_t)r * ld + k;
      if (whole) {
        const lg_u32x4 a = ((const lg_u32x4 LG_GLOBAL*)q)[0], b = ((const lg_u32x4 LG_GLOBAL*)q)[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w[i] = a[i];
          w[4 + i] = b[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t lo = (r < rows && k + 2 * i < ks) ? q[2 * i] : 0u;
          const uint32_t hi = (r < rows && k + 2 * i + 1 < ks) ? q[2 * i + 1] : 0u;
          w[i] = lo | (hi << 16);
        }
      }
    } else {    // rows k0 + (t>>5)*4 + i, columns r0 + (t&31)*4 .. +3 (8-byte aligned: ld a multiple of 4)
      const int r = r0 + (t & 31) * 4, k = k0 + (t >> 5) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t LG_GLOBAL* q = (const uint16_t LG_GLOBAL*)g + (size_t)(k + i) * ld + r;
        if (whole) {
          const lg_u32x2 x = *(const lg_u32x2 LG_GLOBAL*)q;
          w[2 * i] = x[0];
          w[2 * i + 1] = x[1];
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const uint32_t lo = (k + i < ks && r + 2 * j < rows) ? q[2 * j] : 0u;
            const uint32_t hi = (k + i < ks && r + 2 * j + 1 < rows) ? q[2 * j + 1] : 0u;
            w[2 * i + j] = lo | (hi << 16);
          }
        }
      }
    }
  }
  // v <- fl32(v + G), and the largest |v| into mx
  __device__ __forceinline__ void add(float (&v)[16], int gfmt, float& mx) const {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t h = (w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      const float g = gfmt == 0 ? __uint_as_float(h << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)h);
      v[i] = __fadd_rn(v[i], g);
      mx = fmaxf(mx, fabsf(v[i]));
    }
  }
};

// The block's tile (x, y) and batch entry z.  Blocks are dealt to the 8 XCDs
// round-robin by linear id; they are renumbered so that each XCD runs a
// contiguous run of tiles in (x, y, z) order, x fastest: the N tiles of one
// row block, which read the same rows of A, then run at about the same time
// in one XCD and share its L2 (the right product and the CholeskyQR products
// gained 2-4% from this; the split-operand kernel below, whose blocks share
// only small operands, lost 5-12% with it and keeps the plain order).
struct LgBlock {
  int x, y, z;
};
__device__ __forceinline__ LgBlock lg_block() {
  const int gx = gridDim.x, gy = gridDim.y;
  const int total = gx * gy * gridDim.z;
  const int lin = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int xcd = lin & 7, idx = lin >> 3;
  const int base = total >> 3, rem = total & 7;
  const int t = xcd * base + min(xcd, rem) + idx;
  LgBlock b;
  b.x = t % gx;
  b.y = (t / gx) % gy;
  b.z = t / (gx * gy);
  return b;
}

__device__ __forceinline__ uint16_t lg_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace

// The 16-bit G values (laid out as C, ld N) under a 128 x 128 tile in the
// accumulator layout of lg_epilogue below (the four columns of group (a, b, g)
// in two words), read ahead by the split-operand kernel so that their latency
// hides behind its main loop.
typedef uint32_t LgGradTile[2][2][4][2];
__device__ __forceinline__ void lg_read_g(LgGradTile& gw, int M, int N, int m0, int n0, const uint16_t* G) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bool vec = (N & 3) == 0 && ((uintptr_t)G & 7) == 0;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = m0 + wm * 64 + a * 32 + (lane & 31);
        const int col = n0 + wn * 64 + b * 32 + 8 * g + 4 * (lane >> 5);
        const uint16_t LG_GLOBAL* gp = (const uint16_t LG_GLOBAL*)G + (size_t)row * N + col;
        if (vec && row < M && col + 4 <= N) {
          const lg_u32x2 x = *(const lg_u32x2 LG_GLOBAL*)gp;
          gw[a][b][g][0] = x[0];
          gw[a][b][g][1] = x[1];
        } else {
          uint32_t h[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) h[j] = (row < M && col + j < N) ? gp[j] : 0u;
          gw[a][b][g][0] = h[0] | (h[1] << 16);
          gw[a][b][g][1] = h[2] | (h[3] << 16);
        }
      }
}

// The epilogue of a 128 x 128 tile held by four waves of 64 x 64 (2 x 2 MFMA
// blocks), whose MFMAs take the B operand first so that the accumulators
// hold C^T: block (a, b) holds row m0 + wm 64 + a 32 + (lane & 31) and, in
// elements 4g .. 4g + 3, the four consecutive columns n0 + wn 64 + b 32 + 8g
// + 4 (lane / 32) .. + 3; a lane thus reads and writes four columns of a row
// at once.  C (ld ldc, from element coff) = alpha 2^-lab acc (+ beta C with
// READC, fp32 only; with useg, beta fl32(C + G) for the 16-bit G values gw
// that lg_read_g read), written as out_fmt; every read of C is issued before
// any write.  With slot, the block's largest |value| raises *slot.  Every
// thread calls.
template <bool READC>
__device__ __forceinline__ void lg_epilogue(floatx16 (&acc)[2][2], int M, int N, int m0, int n0, int lab,
                                            float alpha, float beta, void* Cp, int ldc, size_t coff, int out_fmt,
                                            unsigned* slot, const LgGradTile& gw, bool useg, int gfmt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bool vec = (N & 3) == 0 && (ldc & 3) == 0 && ((uintptr_t)Cp & 15) == 0 && (coff & 3) == 0;
  const bool readc = READC && out_fmt == 1 && beta != 0.f;
  float LG_GLOBAL* C32 = (float LG_GLOBAL*)Cp + coff;
  uint16_t LG_GLOBAL* C16 = (uint16_t LG_GLOBAL*)Cp + coff;
  float cv[2][2][16];
  if (READC)
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = m0 + wm * 64 + a * 32 + (lane & 31);
        const int col = n0 + wn * 64 + b * 32 + 8 * g + 4 * (lane >> 5);
        const size_t o = (size_t)row * ldc + col;
        if (!readc) {
#pragma unroll
          for (int j = 0; j < 4; ++j) cv[a][b][4 * g + j] = 0.f;
        } else if (vec && row < M && col + 4 <= N) {
          const lg_float4 x = *(const lg_float4 LG_GLOBAL*)(C32 + o);
#pragma unroll
          for (int j = 0; j < 4; ++j) cv[a][b][4 * g + j] = x[j];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) cv[a][b][4 * g + j] = (row < M && col + j < N) ? C32[o + j] : 0.f;
        }
        if (readc && useg) {   // C <- fl32(C + G): the buffer B formed from M and G
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t h = (gw[a][b][g][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
            cv[a][b][4 * g + j] = __fadd_rn(cv[a][b][4 * g + j], gfmt == 0 ? __uint_as_float(h << 16)
                                                                           : (float)__builtin_bit_cast(_Float16, (uint16_t)h));
          }
        }
      }
  float mx = 0.f;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = m0 + wm * 64 + a * 32 + (lane & 31);
        const int col = n0 + wn * 64 + b * 32 + 8 * g + 4 * (lane >> 5);
        const size_t o = (size_t)row * ldc + col;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] = alpha * ldexpf(acc[a][b][4 * g + j], -lab);
          if (readc) v[j] = v[j] + beta * cv[a][b][4 * g + j];
          if (row < M && col + j < N) mx = fmaxf(mx, fabsf(v[j]));
        }
        if (row >= M) continue;
        if (out_fmt == 1) {
          if (vec && col + 4 <= N) {
            *(lg_float4 LG_GLOBAL*)(C32 + o) = lg_float4{v[0], v[1], v[2], v[3]};
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (col + j < N) C32[o + j] = v[j];
          }
        } else {
          uint32_t h[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            h[j] = out_fmt == 0 ? lg_bf16_rne(v[j]) : __builtin_bit_cast(uint16_t, (_Float16)v[j]);
          if (vec && col + 4 <= N) {
            *(lg_u32x2 LG_GLOBAL*)(C16 + o) = lg_u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (col + j < N) C16[o + j] = (uint16_t)h[j];
          }
        }
      }
  if (slot) {   // one atomic per block
    __shared__ float red[4];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    if (tid == 0) {
      const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      if (m > 0.f) atomicMax(slot, __float_as_uint(m));
    }
  }
}

// Row-major C (M x N) = alpha op(A) op(B) for batch entry z of the
// block (lg_block).  A_MODE LG_KC: A is stored M x K (K contiguous, op = N); LG_RC:
// K x M (op = T).  B_MODE LG_KC: B is stored N x K (op = T); LG_RC: K x N
// (op = N).
template <int A_MODE, int B_MODE, bool F16>
__global__ __launch_bounds__(256, 3) void k_lr_gemm(int M, int N, int K, float alpha, const float* const* __restrict__ As,
                                                 int lda, const float* const* __restrict__ Bs, int ldb,
                                                 void* const* __restrict__ Cs, int ldc,
                                                 unsigned* const* __restrict__ amax, int sa, int sb, int sc,
                                                 int out_fmt, int kchunk, int lower_only,
                                                 const uint16_t* const* __restrict__ Gs, int gfmt, int gslot) {
  constexpr int NT = F16 ? 2 : 3;
  __shared__ __attribute__((aligned(16))) uint16_t sA[NT * LG_TERM], sB[NT * LG_TERM];
  // kchunk > 0: K split into chunks, chunk p of product z at batch index
  // z * parts + p, its partial result at C + p M N
  const int parts = kchunk > 0 ? (K + kchunk - 1) / kchunk : 1;
  const LgBlock blk = lg_block();
  const int z = blk.z / parts, part = blk.z - z * parts;
  const int kbeg = part * kchunk, kend = kchunk > 0 ? min(K, kbeg + kchunk) : K;
  if (lower_only && blk.x > blk.y) return;   // a tile wholly above the diagonal
  const float* A = As[z];
  const float* B = Bs[z];
  unsigned* slots = amax[z];
  const int la = F16 ? lg_log2_scale(slots[sa]) : 0, lb = F16 ? lg_log2_scale(slots[sb]) : 0;
  const float scale_a = ldexpf(1.f, la), scale_b = ldexpf(1.f, lb);
  const int m0 = blk.y * LG_TILE, n0 = blk.x * LG_TILE;
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

  LgStage<A_MODE, F16> ga;
  LgStage<B_MODE, F16> gb;
  // with Gs, A is M and the operand is B = fl32(M + G), formed as loaded
  const uint16_t* G = Gs ? Gs[z] : nullptr;
  const bool vecg = (lda & (A_MODE == LG_KC ? 7 : 3)) == 0 && ((uintptr_t)G & 15) == 0;
  LgGrad<A_MODE> gg;
  float bmax = 0.f;
  const int nk = (kend - kbeg + LG_BK - 1) / LG_BK;
  auto load = [&](int k0) {
    ga.load(A, lda, M, kend, m0, k0, veca);
    if (G) gg.load(G, lda, M, kend, m0, k0, vecg);
    gb.load(B, ldb, N, kend, n0, k0, vecb);
  };
  load(kbeg);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();   // every wave is done with the previous stage
    if (G) gg.add(ga.v, gfmt, bmax);
    ga.store(sA, scale_a);
    gb.store(sB, scale_b);
    __syncthreads();
    if (kt + 1 < nk) load(kbeg + (kt + 1) * LG_BK);   // the next stage's loads fly while this one is multiplied
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int chunk = kk * 2 + (lane >> 5);
      uint4 fa[NT][2], fb[NT][2];   // eight 16-bit values each
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int ra = wm * 64 + f * 32 + (lane & 31), rb = wn * 64 + f * 32 + (lane & 31);
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          fa[u][f] = *(const uint4*)(sA + u * LG_TERM + lg_off(ra, chunk));
          fb[u][f] = *(const uint4*)(sB + u * LG_TERM + lg_off(rb, chunk));
        }
      }
      // term products from the smallest weight: F16 hl, lh (2^-11), hh;
      // BF16x3 mm, hl, lh (2^-16), hm, mh (2^-8), hh
      constexpr int NP = F16 ? 3 : 6;
      constexpr int PA[6] = {F16 ? 0 : 1, F16 ? 1 : 0, F16 ? 0 : 2, 0, 1, 0};
      constexpr int PB[6] = {1, F16 ? 0 : 2, 0, 1, 0, 0};
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            if (F16)   // B operand first: the accumulators hold C^T (lg_epilogue)
              acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, fb[PB[p]][b]),
                                                                 __builtin_bit_cast(halfx8, fa[PA[p]][a]), acc[a][b], 0,
                                                                 0, 0);
            else
              acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fb[PB[p]][b]),
                                                                  __builtin_bit_cast(bf16x8, fa[PA[p]][a]), acc[a][b],
                                                                  0, 0, 0);
          }
    }
  }
  const LgGradTile gnone = {};
  lg_epilogue<false>(acc, M, N, m0, n0, la + lb, alpha, 0.f, Cs[z], ldc, (size_t)part * M * N, out_fmt,
              sc >= 0 ? slots + sc : nullptr, gnone, false, 0);
  if (G && gslot >= 0) {   // the largest |B| over this block's share of it
    __shared__ float red[4];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, o, 64));
    if (lane == 0) red[wave] = bmax;
    __syncthreads();
    if (tid == 0) {
      const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      if (m > 0.f) atomicMax(slots + gslot, __float_as_uint(m));
    }
  }
}

void launch_lr_gemm(bool ta, bool tb, bool f16, int m, int n, int k, float alpha, const float* const* A,
                    const float* const* B, void* const* C, unsigned* const* amax, int sa, int sb, int sc,
                    int out_fmt, const uint16_t* const* G, int gfmt, int gslot, int count, hipStream_t s) {
  const int lda = ta ? m : k, ldb = tb ? k : n, ldc = n;
  const dim3 grid((n + LG_TILE - 1) / LG_TILE, (m + LG_TILE - 1) / LG_TILE, count);
#define DION_LRG(AK, BK, F)                                                                                          \
  hipLaunchKernelGGL((k_lr_gemm<AK, BK, F>), grid, dim3(256), 0, s, m, n, k, alpha, A, lda, B, ldb, C, ldc,   \
                     amax, sa, sb, sc, out_fmt, 0, 0, G, gfmt, gslot)
  if (f16) {
    if (!ta && tb) DION_LRG(LG_KC, LG_KC, true);
    else if (!ta && !tb) DION_LRG(LG_KC, LG_RC, true);
    else if (ta && !tb) DION_LRG(LG_RC, LG_RC, true);
    else DION_LRG(LG_RC, LG_KC, true);
  } else {
    if (!ta && tb) DION_LRG(LG_KC, LG_KC, false);
    else if (!ta && !tb) DION_LRG(LG_KC, LG_RC, false);
    else if (ta && !tb) DION_LRG(LG_RC, LG_RC, false);
    else DION_LRG(LG_RC, LG_KC, false);
  }
#undef DION_LRG
}

// ------------------------------------------------ split operands, LDS DMA
// One 16-byte copy per lane from global memory straight into LDS: lane l's
// bytes land at M0 + 16 l.  Completion is tracked by vmcnt, waited for
// explicitly below (the instruction has no register result).
__device__ __forceinline__ void lg_dma16(uint32_t voff, const void* sbase, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void lg_wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// a barrier without __syncthreads' wait for every outstanding copy; the
// wave's own LDS reads are waited for first
__device__ __forceinline__ void lg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}
__device__ __forceinline__ const void* lg_sgpr(const void* p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

// Stages in LDS: two, so that two blocks share a CU (64 KB each).  Products
// with inner dimension r = 256 have eight stages per tile, and a tile's
// prologue and its store-bound epilogue stay exposed unless another block
// runs beside it: four or three stages at one block per CU measured slower
// (31.5 against 24.3 ms for the buffer update) than the register-staged
// kernel, two stages at two blocks faster (22.1 ms).
// With one term per operand (hi only: the update written in bf16, whose
// rounding is eight times the one-term product's) a stage is half as large,
// and four of them fill the same 64 KB.
template <int NT> struct LdCfg {
  static constexpr int STAGES = NT == 2 ? 2 : 4;
  static constexpr int STAGE = 2 * NT * LG_TERM * 2;   // bytes: A hi (, A lo), B hi (, B lo): 8 KB each
  static constexpr int COPIES = STAGE / 1024 / 4;      // 1 KB copies per wave per stage (8 or 4)
};

// C (M x N, row-major, ld N) = alpha A B^T (+ beta C) for product z =
// blockIdx.z, with A (M x K) and B (N x K) split ahead: fp16 hi rows at
// A[z], lo rows rows_a * ldp further on, row length ldp (a multiple of 32),
// rows padded to rows_a (a multiple of 128); zeros in the padding.  Scales
// from slots sa, sb (as k_lr_gemm's F16 operands); sc >= 0 raises slot sc.
// A stage (32 k) of the 128 x 128 tile is 32 KB: four 8 KB term arrays of
// 128 rows x 64 bytes in the swizzled row layout the fragments read.  Each
// wave copies eight 1 KB pieces of it: piece q = 4 i + wave (i < 8) holds
// term q / 8 and rows 16 (q % 8) .. +15, lane l row 16 (q % 8) + l / 4 and
// the chunk whose swizzled position is l % 4.
template <int NT>
__global__ __launch_bounds__(256, 2) void k_lr_gemm_dma(int M, int N, int K, int ldp, int rows_a, int rows_b,
                                                        float alpha, const uint16_t* const* __restrict__ As,
                                                        const uint16_t* const* __restrict__ Bs, float beta,
                                                        void* const* __restrict__ Cs, unsigned* const* __restrict__ amax,
                                                        int sa, int sb, int sc, int out_fmt,
                                                        const uint16_t* const* __restrict__ Gs, int gfmt) {
  constexpr int LD_STAGES = LdCfg<NT>::STAGES, LD_STAGE = LdCfg<NT>::STAGE, LD_COPIES = LdCfg<NT>::COPIES;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[LD_STAGES * LD_STAGE / 2];
  const int z = blockIdx.z;
  unsigned* slots = amax[z];
  const int la = lg_log2_scale(slots[sa]), lb = lg_log2_scale(slots[sb]);
  const int m0 = blockIdx.y * LG_TILE, n0 = blockIdx.x * LG_TILE;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint16_t*)smem);

  // per-lane byte offsets (k = 0) of the eight pieces; the stage's k0 moves the scalar base
  const char* baseA = (const char*)As[z];
  const char* baseB = (const char*)Bs[z];
  uint32_t voff[LD_COPIES];
#pragma unroll
  for (int i = 0; i < LD_COPIES; ++i) {
    const int q = 4 * i + wave, term = q / 8;   // term array: operand term / NT, its term % NT
    const int row = 16 * (q % 8) + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    const int r0 = term < NT ? m0 : n0;
    const size_t tstride = (size_t)(term < NT ? rows_a : rows_b) * ldp;
    voff[i] = (uint32_t)((((size_t)(term % NT) * tstride) + (size_t)(r0 + row) * ldp + 8 * c) * 2);
  }
  auto issue = [&](int kt) {   // the copies of stage kt into buffer kt % LD_STAGES
    const uint32_t st = lds0 + (uint32_t)((kt % LD_STAGES) * LD_STAGE);
#pragma unroll
    for (int i = 0; i < LD_COPIES; ++i) {
      const int q = 4 * i + wave;
      const char* b = (q / 8 < NT ? baseA : baseB) + (size_t)kt * LG_BK * 2;
      lg_dma16(voff[i], lg_sgpr(b), (uint32_t)__builtin_amdgcn_readfirstlane(st + q * 1024));
    }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  const int nk = K / LG_BK;   // K = ldp, a multiple of 32
  // G (the buffer update's B = fl32(C + G)) read first: the loads complete
  // while the main loop runs (the first stage's wait covers them)
  const bool pg = Gs && out_fmt == 1 && beta != 0.f;
  LgGradTile gw;
  if (pg) lg_read_g(gw, M, N, m0, n0, Gs[z]);
#pragma unroll
  for (int kt = 0; kt < LD_STAGES - 1; ++kt)
    if (kt < nk) issue(kt);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed once at most the later stages already issued are outstanding
    const int later = min(nk, kt + LD_STAGES - 1) - kt - 1;
    if (later >= 2) lg_wait_vmcnt<2 * LD_COPIES>();   // at most LD_STAGES - 2 = 2
    else if (later == 1) lg_wait_vmcnt<LD_COPIES>();
    else lg_wait_vmcnt<0>();
    lg_barrier();   // every wave's copies of stage kt have landed, and every wave is done with stage kt - 1
    if (kt + LD_STAGES - 1 < nk) issue(kt + LD_STAGES - 1);   // into stage kt - 1's buffer
    const uint16_t* sbuf = smem + (kt % LD_STAGES) * (LD_STAGE / 2);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int chunk = kk * 2 + (lane >> 5);
      halfx8 fa[NT][2], fb[NT][2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int ra = wm * 64 + f * 32 + (lane & 31), rb = wn * 64 + f * 32 + (lane & 31);
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          fa[u][f] = *(const halfx8*)(sbuf + u * LG_TERM + lg_off(ra, chunk));
          fb[u][f] = *(const halfx8*)(sbuf + (NT + u) * LG_TERM + lg_off(rb, chunk));
        }
      }
      // hl, lh (two terms), then hh
      if constexpr (NT == 2) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[1][b], fa[0][a], acc[a][b], 0, 0, 0);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[0][b], fa[1][a], acc[a][b], 0, 0, 0);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[0][b], fa[0][a], acc[a][b], 0, 0, 0);
    }
  }
  lg_epilogue<true>(acc, M, N, m0, n0, la + lb, alpha, beta, Cs[z], N, 0, out_fmt, sc >= 0 ? slots + sc : nullptr,
                    gw, pg, gfmt);
}

void launch_lr_gemm_split(int m, int n, int k, int ldp, int rows_a, int rows_b, float alpha, const uint16_t* const* A,
                          const uint16_t* const* B, float beta, void* const* C, unsigned* const* amax, int sa, int sb,
                          int sc, int out_fmt, const uint16_t* const* G, int gfmt, int count, hipStream_t s) {
  (void)k;
  const dim3 grid((n + LG_TILE - 1) / LG_TILE, (m + LG_TILE - 1) / LG_TILE, count);
  if (out_fmt == 0)   // a bf16 result: the hi terms alone
    hipLaunchKernelGGL(k_lr_gemm_dma<1>, grid, dim3(256), 0, s, m, n, ldp, ldp, rows_a, rows_b, alpha, A, B, beta, C,
                       amax, sa, sb, sc, out_fmt, G, gfmt);
  else
    hipLaunchKernelGGL(k_lr_gemm_dma<2>, grid, dim3(256), 0, s, m, n, ldp, ldp, rows_a, rows_b, alpha, A, B, beta, C,
                       amax, sa, sb, sc, out_fmt, G, gfmt);
}

void launch_lr_gram(int rows, int r, const float* const* F, float* const* S, unsigned* const* amax, int sf, int count,
                    hipStream_t s) {
  const int parts = (rows + LR_GRAM_CHUNK - 1) / LR_GRAM_CHUNK;
  const dim3 grid((r + LG_TILE - 1) / LG_TILE, (r + LG_TILE - 1) / LG_TILE, count * parts);
  hipLaunchKernelGGL((k_lr_gemm<LG_RC, LG_RC, true>), grid, dim3(256), 0, s, r, r, rows, 1.f, F, r, F, r,
                     (void* const*)S, r, amax, sf, sf, -1, 1, LR_GRAM_CHUNK, 1, nullptr, 0, -1);
}

// Split a batch of row-major fp32 matrices (rows x k) into fp16 hi and lo
// rows of length ldp (k rounded up to 32) at dst, rows padded to rows_pad (a
// multiple of 128), zeros in the padding, lo rows_pad * ldp after hi; with
// the scale that slot `slot` gives: the F16 operand format above.  Grid
// (blocks over rows_pad * ldp / 8, count), 8 values per thread.
__global__ __launch_bounds__(256) void k_lr_split16(const float* const* __restrict__ src, uint16_t* const* __restrict__ dst,
                                                    int rows, int rows_pad, int k, int ldp,
                                                    unsigned* const* __restrict__ amax, int slot) {
  const int z = blockIdx.y;
  const int64_t e8 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cpr = ldp / 8;
  if (e8 >= (int64_t)rows_pad * cpr) return;
  const int r = (int)(e8 / cpr), k0 = (int)(e8 - (int64_t)r * cpr) * 8;
  const float scale = ldexpf(1.f, lg_log2_scale(amax[z][slot]));
  const float* p = src[z] + (size_t)r * k + k0;
  float v[8];
  if (r >= rows) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  } else if (k0 + 8 <= k && (k & 3) == 0 && ((uintptr_t)src[z] & 15) == 0) {
    *(float4*)&v[0] = *(const float4*)p;
    *(float4*)&v[4] = *(const float4*)(p + 4);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = k0 + i < k ? p[i] : 0.f;
  }
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t a[3], b[3];
    lg_split<true>(v[2 * i], scale, a);
    lg_split<true>(v[2 * i + 1], scale, b);
    h[i] = a[0] | (b[0] << 16);
    l[i] = a[1] | (b[1] << 16);
  }
  uint16_t* d = dst[z] + (size_t)r * ldp + k0;
  *(uint4*)d = make_uint4(h[0], h[1], h[2], h[3]);
  *(uint4*)(d + (size_t)rows_pad * ldp) = make_uint4(l[0], l[1], l[2], l[3]);
}

void launch_lr_split16(const float* const* src, uint16_t* const* dst, int rows, int rows_pad, int k, int ldp,
                       unsigned* const* amax, int slot, int count, hipStream_t s) {
  const int64_t n8 = (int64_t)rows_pad * (ldp / 8);
  if (n8 > 0 && count > 0)
    hipLaunchKernelGGL(k_lr_split16, dim3((unsigned)((n8 + 255) / 256), count), dim3(256), 0, s, src, dst, rows,
                       rows_pad, k, ldp, amax, slot);
}

}  // namespace dion
