// Internal structures shared by the host planner and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dion {

// Every operand buffer in the workspace has both dimensions padded to a
// multiple of PAD (the largest GEMM tile), and the padding holds zeros, so the
// MFMA main loops never need bounds checks.
constexpr int PAD = 256;

inline __host__ __device__ int pad_up(int x) { return (x + PAD - 1) / PAD * PAD; }

// Element offset of (r, c) in an fp16 workspace matrix with ld columns (MFMA16
// path; ld a multiple of 32, rows a multiple of 256).  The matrix is stored
// panel-blocked: blocks of 256 rows x 32 columns, each contiguous (8192
// elements), ordered by row-block, then column-block.  Inside a block, row r
// holds its 32 columns as four 8-element chunks, chunk j at position
// j ^ ((r / 4) & 3).  One K-stage (32 columns) of a GEMM tile's operand is
// then one contiguous run of whole cache lines, and a linear global -> LDS
// copy of it lands in the XOR-swizzled layout the MFMA fragment reads want.
// 8-column groups starting at a multiple of 8 stay contiguous.  FP64 path
// buffers are plain row-major.
inline __host__ __device__ size_t blk_off(int r, int c, int ld) {
  return ((size_t)(r >> 8) * (size_t)(ld >> 5) + (size_t)(c >> 5)) * 8192u + (size_t)(r & 255) * 32u +
         (size_t)(((((unsigned)c >> 3) & 3u) ^ (((unsigned)r >> 2) & 3u)) << 3) + (size_t)(c & 7);
}

// Buffer slots of a matrix's workspace region.
enum Slot : int {
  SLOT_X = 0,   // [m_pad][n_pad] hi: Gram (SYRK) operand
  SLOT_XT0 = 1, // [n_pad][m_pad] x terms: apply operand (X0^T from the pack)
  SLOT_XT1 = 2, // [n_pad][m_pad] x terms: iterate of odd-numbered restarts
  SLOT_XTE = 3, // iterate of even-numbered restarts: XT0's buffer, or XT1's for
                // matrices that restart from X0 (their X0^T must survive)
  SLOT_MM0 = 4, // m_pad x m_pad buffers: G, P, T, Q roles rotate over four;
  SLOT_MM1 = 5, // two more hold the accumulated factor and its transpose when
  SLOT_MM2 = 6, // some matrix restarts from X0
  SLOT_MM3 = 7,
  SLOT_MM4 = 8,
  SLOT_MM5 = 9,
  N_SLOTS = 10
};

// Per-matrix descriptor (device copy in the workspace).
struct MatDesc {
  const void* M;      // input (R x C), or the fp32 momentum buffer in step mode
  void* out;          // output (R x C)
  const void* grad;   // step mode: gradient (R x C)
  void* buf[N_SLOTS]; // workspace buffers (fp16 or fp64 elements)
  int64_t row0;       // first global row (into keys / flags)
  int64_t sel0;       // first entry of this matrix in the idx array
  int R, C;           // stored shape
  int k;              // selected rows
  int m, n;           // Gram side and long side (m <= n)
  int m_pad, n_pad;   // padded
  int tall;           // 1 if the selected block is tall (k > C): X = S^T
  float upd_alpha;    // weight-update mode: W <- W * keep - upd_alpha * update
};

// Per-matrix scalars written by the device (selection / normalization).
struct MatScalars {
  double nu2;         // ||S||_F^2
  double x0_alpha64;  // X0 = stored operand * x0_alpha (= 2^-e / nu, 0 if nu = 0)
  float x0_alpha;     // the same in fp32
  int e;              // stored operand = S * 2^e (0 on the FP64 path)
};

// Epilogue kinds of the GEMM kernels.
enum Epi : int {
  EPI_SYM = 0,   // symmetric output: write the upper tile and its mirror
  EPI_POLY = 1,  // symmetric output P = a I + b G + c acc (G read from aux)
  EPI_RECT = 2,  // rectangular internal output
  EPI_OUT = 3,   // final output rows -> out[rowmap[r]] (masked to valid)
  EPI_RECT_T = 4 // EPI_RECT, plus the transposed hi term into aux (the Gram operand)
};

// Arguments of one GEMM phase: C = alpha * A B^T over a list of tiles.
struct PhaseArgs {
  int a_slot, b_slot, c_slot, aux_slot;
  int a_rows_is_n;   // rows of A: 1 -> n_pad, 0 -> m_pad
  int b_rows_is_n;   // rows of B
  int k_is_n;        // reduction length: 1 -> n_pad, 0 -> m_pad
  int alpha_pow;     // alpha *= x0_alpha^alpha_pow (per matrix)
  float alpha;       // scale applied to the accumulator
  float out_scale;   // scale of the stored output (fp16 power of two)
  float poly_a, poly_b, poly_c;  // EPI_POLY coefficients
  float aux_inv_scale;           // EPI_POLY: G = stored aux * aux_inv_scale
  int aux_lo;                    // EPI_POLY (MFMA16): 1 -> G = hi + lo, 0 -> hi only
  int out_fp32;      // EPI_OUT: 1 -> fp32 output, 0 -> 16-bit (bf16, or fp16 when out_f16)
  int out_f16;       // EPI_OUT: 16-bit output in fp16 rather than bf16
  int out_rows_are_m;  // EPI_OUT: 1 -> product rows index the m side
  int out_lo;        // fp16 outputs: 1 -> store the lo term too, 0 -> hi only (no reader needs lo)
  int out_update;    // EPI_OUT: 1 -> out is the weight W, updated as W <- W * upd_keep - upd_alpha * value
  float upd_keep;    // EPI_OUT weight update: 1 - decoupled weight decay
  const MatScalars* scalars;
  const int* idx;      // selected rows (global), NULL when row_frac == 1
};

// One grouped launch: the matrices it covers and the prefix of their tile counts.
struct GemmLaunch {
  const MatDesc* descs;
  const int* mats;
  const int* prefix;
  int nmat;
  int total;           // tiles
  const int* ranges;   // 9 ints: XCD x runs tiles [ranges[x], ranges[x+1])
  int grid;            // 8 * the largest range
};

}  // namespace dion
