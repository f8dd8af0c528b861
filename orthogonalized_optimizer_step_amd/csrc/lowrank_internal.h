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
  float* S;          // r x r  Gram of the factor being orthogonalized
  float* Linv;       // r x r  inverse of its Cholesky factor (lower)
  double* A64;       // r x r  fp64 scratch of the factorization
  float* D;          // R x C  fp32 update before the cast (or == out)
  int64_t elems;     // R * C
  int64_t blk0;      // first block of this matrix in the element-wise launches
  int R, C, r;
  int pad_;
};

// element-wise launches: 256 threads x 8 elements per block
constexpr int LR_BLOCK_ELEMS = 2048;
// ranks up to this factor their Gram matrix in registers (k_lr_cholinv_reg)
constexpr int LR_REG_RMAX = 256;

void launch_lr_accumulate(const LrDesc* d, int nmat, int64_t blocks, int grad_fmt, hipStream_t s);
void launch_lr_cast(const LrDesc* d, int nmat, int64_t blocks, int out_fmt, hipStream_t s);
// shift > 0: factor S + shift * (largest diagonal entry of S) * I (the first,
// shifted pass of shifted CholeskyQR3)
void launch_lr_cholinv(const LrDesc* d, int nmat, bool any_small, bool any_large, float shift, hipStream_t s);
void launch_lr_colnorm(const LrDesc* d, int nmat, hipStream_t s);

}  // namespace dion
