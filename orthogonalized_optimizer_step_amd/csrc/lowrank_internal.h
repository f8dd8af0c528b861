// Internal declarations of the low-rank (Dion / Orth-Dion) step: one
// descriptor per matrix, shared by the host planner (lowrank.cpp) and the
// kernels (lowrank_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace dion {

struct LrDesc {
  float* M;          // R x C fp32 buffer (in place)
  const void* G;     // R x C gradient
  float* Q;          // C x r right factor (in: previous, out: new)
  void* out;         // R x C update
  float* X;          // R x r  P = orth(B Q)
  float* Y;          // R x r  B Q, then a CholeskyQR intermediate
  float* W;          // C x r  right factor before normalization
  float* W2;         // C x r  CholeskyQR intermediate of W
  float* S;          // r x r  Gram of the factor being orthogonalized, as
                     // parts_R or parts_C partial sums (r x r each, K split)
  float* Linv;       // r x r  inverse of its Cholesky factor (lower)
  double* A64;       // r x r  fp64 scratch of the factorization
  unsigned* amax;    // LS_N slots: the largest |value| of each operand the
                     // GEMMs read (fp32 bits; zero at the start of a call)
  int64_t elems;     // R * C
  int64_t blk0;      // first block of this matrix in the element-wise launches
  int R, C, r;
  int parts_R, parts_C;   // K chunks of the Gram of an R x r / C x r factor
  int pad_;
};

// Operands of the step's products, each with a slot for its largest |value|,
// from which the GEMM that reads it takes its fp16 scale.  The producer of
// an operand raises its slot (atomicMax on the bits of a non-negative float):
// the accumulation for B (through per-block maxima), the GEMM epilogues for
// their outputs, the factorization for L^-1.  (The power product B Q takes
// unscaled bf16 terms, so the incoming Q needs none.)  CholeskyQR3 of
// the power product: pass p reads F_{p-1} (F_-1 = Y) and L_p, writes F_p
// (F_2 = P); of the right factor: pass p reads G_{p-1} (G_-1 = W) and L_{3+p},
// writes G_p (G_2 = the new Q).  Dion's column normalization bounds the new
// Q by one: its slot starts at 1.
enum LrSlot {
  LS_B, LS_Y, LS_W,
  LS_L0, LS_L1, LS_L2, LS_L3, LS_L4, LS_L5,
  LS_F0, LS_F1, LS_F2, LS_G0, LS_G1, LS_G2,
  LS_N
};

// element-wise launches: 256 threads x 8 elements per block
constexpr int LR_BLOCK_ELEMS = 2048;
// ranks up to this factor their Gram matrix in registers (k_lr_cholinv_reg)
constexpr int LR_REG_RMAX = 256;

// blocks per matrix of k_lr_absmax and of k_lr_gram_sum
constexpr int LR_ABSMAX_SPLIT = 16;
constexpr int LR_SUM_SPLIT = 256;
// rows of the factor per K chunk of a CholeskyQR Gram product
constexpr int LR_GRAM_CHUNK = 1024;

// B = fl32(M + G) in place, each block's largest |B| to blockmax (one float
// per element-wise block); then the LS_B slot from those
void launch_lr_accumulate(const LrDesc* d, int nmat, int64_t blocks, int grad_fmt, float* blockmax, hipStream_t s);
void launch_lr_absmax(const LrDesc* d, int nmat, const float* blockmax, hipStream_t s);
// S is the sum of the parts_R (rows_are_R) or parts_C partial Grams, added
// in order in fp64 into A64 (k_lr_gram_sum); shift > 0: factor S + shift * (largest diagonal entry of S) * I
// (the first, shifted pass of shifted CholeskyQR3); the largest |entry| of
// L^-1 raises slot `amax_slot`
void launch_lr_cholinv(const LrDesc* d, int nmat, bool any_small, bool any_large, bool rows_are_R, float shift,
                       int amax_slot, hipStream_t s);
void launch_lr_colnorm(const LrDesc* d, int nmat, hipStream_t s);
// Row-major C (m x n) = alpha op(A) op(B) over `count` products (device
// pointer arrays; amax: each product's matrix's LS_N slots), on two-term
// fp16 operands (f16) or three-term bf16 ones.  The fp16 operands' scales
// come from slots sa and sb; sc >= 0 raises slot sc with the result's
// largest |value|.  out_fmt: 1 fp32, 0 bf16 or 2 fp16 (round to nearest even).
// With G (16-bit gradients laid out as A, gfmt 0 bf16 or 2 fp16), the A
// operand is fl32(A + G), and gslot >= 0 raises slot gslot with its largest
// |value|.
void launch_lr_gemm(bool ta, bool tb, bool f16, int m, int n, int k, float alpha, const float* const* A,
                    const float* const* B, void* const* C, unsigned* const* amax, int sa, int sb, int sc,
                    int out_fmt, const uint16_t* const* G, int gfmt, int gslot, int count, hipStream_t s);
// C (m x n, ld n) = alpha A B^T + beta C with both operands split ahead by
// launch_lr_split16: A as m rows (padded to rows_a) and B as n rows (padded
// to rows_b) of k values (fp16 hi and lo, row length ldp); out_fmt 1 fp32
// (with beta), 0 bf16 or 2 fp16 (beta must be 0).  With G (16-bit, laid out
// as C), beta C is beta fl32(C + G).  A bf16 result reads the hi terms only
// (one product, k_lr_gemm_dma<1>): its rounding, 2^-9 relative, is eight
// times the one-term product's; the others read both terms (three products).
void launch_lr_gemm_split(int m, int n, int k, int ldp, int rows_a, int rows_b, float alpha, const uint16_t* const* A,
                          const uint16_t* const* B, float beta, void* const* C, unsigned* const* amax, int sa, int sb,
                          int sc, int out_fmt, const uint16_t* const* G, int gfmt, int count, hipStream_t s);
// The Gram F^T F of `count` row-major fp32 factors F (rows x r, F16 terms
// with the scale of slot sf): the rows split into chunks of LR_GRAM_CHUNK,
// chunk p's r x r partial written at S + p r r (only the tiles on or below
// the diagonal, all that the factorization reads).
void launch_lr_gram(int rows, int r, const float* const* F, float* const* S, unsigned* const* amax, int sf,
                    int count, hipStream_t s);
// Split `count` row-major fp32 matrices (rows x k) with the scale of slot
// `slot` into fp16 hi and lo rows of length ldp = k rounded up to 32, rows
// padded to rows_pad = rows rounded up to 128 (zeros in the padding; lo
// after hi): rows_pad * ldp * 4 bytes at each dst.
void launch_lr_split16(const float* const* src, uint16_t* const* dst, int rows, int rows_pad, int k, int ldp,
                       unsigned* const* amax, int slot, int count, hipStream_t s);

}  // namespace dion
