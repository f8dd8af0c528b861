// Grouped (megabatched) GEMM kernels of the Gram Newton-Schulz iteration.
//
// Every product of the iteration is C = alpha * A * B^T with both operands
// stored row-major with the reduction dimension contiguous ("NT"):
//   Gram        G = X X^T            (X: m x n)            symmetric output
//   m x m chain G*G, P*T^T           (symmetric, commuting) symmetric output
//               P*G, P*Q^T           symmetric output for two-term operands,
//                                    full (rectangular) for one-term ones
//   apply       X'^T = X^T Q         (X^T: n x m, Q: m x m) rectangular
//   final       out = Q X  or  X^T Q, scattered to the selected output rows
// Symmetric outputs are computed on upper-triangle tiles only and written
// twice (tile and mirror), the triangular scheduling and transpose epilogue
// the Dion3 summary describes for its symmetric GEMM kernels (方法 / 核心模块,
// CuteDSL bullet); the polynomial P = aI + bG + cG^2 is fused into the G*G
// epilogue (the same bullet's fused GEMM + add).
//
// One launch covers every matrix of the batch: blocks map to (matrix, tile)
// through a prefix table of tile counts, and block ids are remapped so that
// each of the 8 XCDs (blocks are dealt to XCDs round-robin) walks a
// contiguous run of tiles, keeping shared operand panels in its own L2.
//
// MFMA16 path: fp16 operands with power-of-two scales, v_mfma_f32_32x32x16_f16
// with fp32 accumulation; an operand may carry two terms (hi + lo, the lo
// term being the fp16 rounding of the residual), in which case the products
// hi*hi + hi*lo + lo*hi are accumulated.  FP64 path: plain fp64 FMA tiles.
#include <utility>

#include "dion_internal.h"

namespace dion {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Pointers read from descriptors are generic; loads through them become flat
// loads, which count against the LDS wait counter too and would make every
// LDS fragment wait also wait for the in-flight HBM loads.  Casting to the
// global address space gives global loads tracked by vmcnt only.
#define DION_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const T DION_GLOBAL* to_global(const T* p) {
  return (const T DION_GLOBAL*)p;
}
template <typename T>
__device__ __forceinline__ T DION_GLOBAL* to_global_w(T* p) {
  return (T DION_GLOBAL*)p;
}

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ int find_segment(const int* prefix, int n, int t) {
  int lo = 0, hi = n;  // prefix[lo] <= t < prefix[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (prefix[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Blocks are dealt to the 8 XCDs round-robin; block b runs tile
// ranges[x] + b / 8 of the contiguous range [ranges[x], ranges[x+1]) of XCD
// x = b % 8, so the tiles an XCD runs at once share operand panels in its
// L2.  The host sizes the ranges to equal work (tiles weighted by their
// reduction depth), and launches 8 * (largest range) blocks; the rest exit.
__device__ __forceinline__ int range_tile(const int* __restrict__ ranges, int b) {
  const int x = b & 7;
  const int t = ranges[x] + (b >> 3);
  return t < ranges[x + 1] ? t : -1;
}

// Tile order within a matrix: bands of GROUP tile-rows, each band walked
// column by column, so the ~32 tiles an XCD runs at once share a few operand
// panels (K-slices of them stay in that XCD's L2).  Symmetric outputs use the
// same banding restricted to the upper triangle (ti <= tj).
constexpr int GROUP = 8;

__device__ __forceinline__ void decode_tile(bool sym, int local, int arows, int brows, int bm,
                                            int& ti, int& tj) {
  const int TM = arows / bm, TN = brows / bm;
  if (sym) {
    int r0 = 0;
    while (r0 < TM) {
      const int r1 = min(TM, r0 + GROUP);
      int band = 0;  // tiles of rows [r0, r1) with tj >= ti
      for (int i = r0; i < r1; ++i) band += TN - i;
      if (local < band) {
        for (int j = r0;; ++j) {
          const int cnt = min(j + 1, r1) - r0;  // rows i in [r0, r1) with i <= j
          if (local < cnt) { ti = r0 + local; tj = j; return; }
          local -= cnt;
        }
      }
      local -= band;
      r0 = r1;
    }
    ti = tj = 0;  // unreachable for local < T(T+1)/2
  } else {
    const int band_rows = GROUP;
    const int band = local / (band_rows * TN);
    const int r0 = band * band_rows;
    const int rows = min(band_rows, TM - r0);
    const int l = local - band * band_rows * TN;
    tj = l / rows;
    ti = r0 + l % rows;
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Storage of internal matrices: fp16 hi/lo pairs (term stride apart) or fp64.
template <typename ST> struct Store;
template <> struct Store<_Float16> {
  __device__ static void put(void* base, size_t term_stride, size_t off, float v) {
    _Float16 h = (_Float16)v;
    _Float16 l = (_Float16)(v - (float)h);
    ((_Float16*)base)[off] = h;
    ((_Float16*)base)[off + term_stride] = l;
  }
  __device__ static float get(const void* base, size_t term_stride, size_t off) {
    const _Float16* p = (const _Float16*)base;
    return (float)p[off] + (float)p[off + term_stride];
  }
};
template <> struct Store<double> {
  __device__ static void put(void* base, size_t, size_t off, double v) { ((double*)base)[off] = v; }
  __device__ static double get(const void* base, size_t, size_t off) { return ((const double*)base)[off]; }
};

// Epilogue for one accumulator element at tile-local (r, c) of tile (ti, tj).
template <int EPI, typename ST, typename AT>
__device__ __forceinline__ void epilogue_elem(const MatDesc& d, const PhaseArgs& pa, int arows,
                                              int brows, int ti, int tj, int bm, int r, int c,
                                              AT acc, AT alpha) {
  const int gi = ti * bm + r, gj = tj * bm + c;
  if (EPI == EPI_SYM || EPI == EPI_POLY) {
    const bool diag = (ti == tj);
    if (diag && c < r) return;  // the diagonal tile writes its upper half (+ mirror)
    const int ld = arows;       // square
    const size_t ts = (size_t)ld * ld;
    AT v;
    if (EPI == EPI_POLY) {
      if (gi >= d.m || gj >= d.m) {
        v = 0;  // keep the zero padding (the identity term would fill it)
      } else {
        const AT g = (AT)Store<ST>::get(d.buf[pa.aux_slot], ts, (size_t)gi * ld + gj) * (AT)pa.aux_inv_scale;
        v = (AT)pa.poly_b * g + (AT)pa.poly_c * (acc * alpha);
        if (gi == gj) v += (AT)pa.poly_a;
        v *= (AT)pa.out_scale;
      }
    } else {
      v = acc * alpha;
    }
    Store<ST>::put(d.buf[pa.c_slot], ts, (size_t)gi * ld + gj, v);
    if (gi != gj) Store<ST>::put(d.buf[pa.c_slot], ts, (size_t)gj * ld + gi, v);
  } else if (EPI == EPI_RECT) {
    const size_t ts = (size_t)arows * brows;
    Store<ST>::put(d.buf[pa.c_slot], ts, (size_t)gi * brows + gj, acc * alpha);
  } else {  // EPI_OUT
    const int rows_valid = pa.out_rows_are_m ? d.m : d.n;
    const int cols_valid = pa.out_rows_are_m ? d.n : d.m;
    if (gi >= rows_valid || gj >= cols_valid) return;
    const int orow = pa.idx ? pa.idx[d.sel0 + gi] : gi;
    const size_t o = (size_t)orow * d.C + gj;
    const float v = (float)(acc * alpha);
    if (pa.out_fp32) ((float*)d.out)[o] = v;
    else if (pa.out_f16) ((_Float16*)d.out)[o] = (_Float16)v;
    else ((uint16_t*)d.out)[o] = f32_to_bf16_rne(v);
  }
}

template <typename AT>
__device__ __forceinline__ AT phase_alpha(const MatDesc& d, const PhaseArgs& pa, int mi) {
  AT a = (AT)pa.alpha;
  if (pa.alpha_pow > 0) {
    const AT f = sizeof(AT) == 8 ? (AT)pa.scalars[mi].x0_alpha64 : (AT)pa.scalars[mi].x0_alpha;
    a *= f;
    if (pa.alpha_pow > 1) a *= f;
  }
  return a;
}

// ------------------------------------------------- strip-staged epilogue
// Each wave turns its (WT x WT) sub-tile into stores 32 rows ("a strip") at a
// time: the strip's fp32 values go to LDS row-major, then leave as 16-byte
// chunks of 8 consecutive columns.  The transposed copy (the mirror of a
// symmetric output, or X from X^T after a restart) needs no staging: in the
// accumulator layout a lane holds 4 consecutive rows of one column, which are
// 4 consecutive columns of a transposed row, so it leaves straight from
// registers (8-byte stores, or 16-byte ones after an exchange between lanes l
// and l + 32).  A diagonal tile of a symmetric output is written
// whole by the direct stores (both of its triangles are computed) and has no
// mirror, so no store is masked except at the valid edge of the final output.
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ constexpr int epi_wave_bytes(int wt) {
  return 32 * (wt + 8) * 4;   // row-major strip 32 x (wt + 8) floats
}

__device__ __forceinline__ void split8(const float* v, half8v& h, half8v& l) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const _Float16 x = (_Float16)v[i];
    h[i] = x;
    l[i] = (_Float16)(v[i] - (float)x);
  }
}

// 8 consecutive columns [col0, col0+8) of row `row` (col0 a multiple of 8) of
// a panel-blocked fp16 hi/lo matrix (ld columns, lo term `ts` elements after
// hi; the lo term only if `lo`); elements with !mask skipped.
__device__ __forceinline__ void store8_split(_Float16* base, size_t ts, int ld, int row, int col0,
                                             const float* v, unsigned mask, bool lo) {
  half8v h, l;
  split8(v, h, l);
  const size_t off = blk_off(row, col0, ld);
  _Float16 DION_GLOBAL* g = to_global_w(base);
  if (mask == 0xFFu) {
    *(half8v DION_GLOBAL*)(g + off) = h;
    if (lo) *(half8v DION_GLOBAL*)(g + off + ts) = l;
  } else if (mask) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (mask >> i & 1u) {
        g[off + i] = h[i];
        if (lo) g[off + ts + i] = l[i];
      }
  }
}

// 8 consecutive columns of row `row` of a panel-blocked matrix, hi term only.
__device__ __forceinline__ void store8_hi(_Float16* base, int ld, int row, int col0, const float* v) {
  half8v h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (_Float16)v[i];
  *(half8v DION_GLOBAL*)(to_global_w(base) + blk_off(row, col0, ld)) = h;
}

// The epilogue's LDS staging area is private to each wave, and a wave's LDS
// operations execute in issue order, so handing values between its lanes
// through LDS needs only to keep the compiler from reordering the accesses.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("" : : : "memory"); }

// One strip (compile-time index A) of the epilogue.
template <int BM, int EPI, int F, int A, bool DIAG>
__device__ __forceinline__ void epilogue_strip(const MatDesc& d, const PhaseArgs& pa, float alpha, int arows,
                                               int brows, int ti, int tj, int wm, int wn, int lane,
                                               const floatx16 (&acc)[F][F], float* st) {
  constexpr int WT = F * 32;
  constexpr int SROW = WT + 8;   // row-major strip stride (floats)
  constexpr bool SYMO = (EPI == EPI_SYM || EPI == EPI_POLY);
  constexpr int a = A;
  // the transposed copy: mirror of an off-diagonal symmetric tile, or X (hi)
  constexpr bool TRANS = (SYMO && !DIAG) || EPI == EPI_RECT_T;
  const int row_base = ti * BM + wm * WT;  // global row of the sub-tile
  const int col_base = tj * BM + wn * WT;  // global col of the sub-tile
  _Float16* C = (_Float16*)d.buf[pa.c_slot];
  const size_t cts = SYMO ? (size_t)arows * arows : (size_t)arows * brows;
  const int cld = SYMO ? arows : brows;

  {
    // ---- values of strip a, in the accumulator layout
    float v[F][16];
    if (EPI == EPI_POLY) {
      // G[gi][gj] for 4 consecutive rows = G[gj][gi..gi+3] (G is symmetric);
      // every load of the strip is issued before any store of it.  The lo
      // term is read only when the product runs on two-term operands.
      const _Float16* G = (const _Float16*)d.buf[pa.aux_slot];
      const bool with_lo = pa.aux_lo != 0;
      half4 gh[F][4], gl[F][4];
#pragma unroll
      for (int b = 0; b < F; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int gi = row_base + a * 32 + g * 8 + (lane >> 5) * 4;
          const int gj = col_base + b * 32 + (lane & 31);
          const size_t off = blk_off(gj, gi, arows);   // 4 contiguous elements (gi % 4 == 0)
          gh[b][g] = *to_global((const half4*)(G + off));
          gl[b][g] = with_lo ? *to_global((const half4*)(G + off + cts)) : half4{0, 0, 0, 0};
        }
#pragma unroll
      for (int b = 0; b < F; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int gi = row_base + a * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
          const int gj = col_base + b * 32 + (lane & 31);
          const float g = ((float)gh[b][e >> 2][e & 3] + (float)gl[b][e >> 2][e & 3]) * pa.aux_inv_scale;
          float x = pa.poly_b * g + pa.poly_c * (acc[a][b][e] * alpha);
          if (gi == gj) x += pa.poly_a;
          x *= pa.out_scale;
          v[b][e] = (gi < d.m && gj < d.m) ? x : 0.f;  // keep the zero padding
        }
    } else {
#pragma unroll
      for (int b = 0; b < F; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) v[b][e] = acc[a][b][e] * alpha;
    }

    // ---- row-major strip -> direct stores
#pragma unroll
    for (int b = 0; b < F; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        st[((e >> 2) * 8 + (lane >> 5) * 4 + (e & 3)) * SROW + b * 32 + (lane & 31)] = v[b][e];
    wave_lds_sync();
    constexpr int CPR = WT / 8;  // chunks per strip row
#pragma unroll
    for (int q0 = 0; q0 < 32 * CPR; q0 += 64) {
      const int q = q0 + lane;
      const int rr = q / CPR, c0 = (q % CPR) * 8;
      float w[8];
      *(float4*)&w[0] = *(const float4*)&st[rr * SROW + c0];
      *(float4*)&w[4] = *(const float4*)&st[rr * SROW + c0 + 4];
      const int gi = row_base + a * 32 + rr, gj0 = col_base + c0;
      if (EPI == EPI_OUT) {
        const int rows_valid = pa.out_rows_are_m ? d.m : d.n;
        const int cols_valid = pa.out_rows_are_m ? d.n : d.m;
        if (gi < rows_valid && gj0 < cols_valid) {
          const int orow = pa.idx ? *to_global(pa.idx + d.sel0 + gi) : gi;
          const size_t o = (size_t)orow * d.C + gj0;
          const bool full = gj0 + 8 <= cols_valid;
          // output (and weight) accesses through global pointers: flat ones
          // would also count against the LDS wait counter of the next strip
          if (pa.out_update) {
            // the weight update: W <- fl32(fl32(W * keep) - fl32(alpha * u)),
            // rounded to W's dtype below (u = this fp32 output)
            float cur[8];
            if (pa.out_fp32) {
              const float DION_GLOBAL* wp = to_global((const float*)d.out) + o;
              if (full && ((uintptr_t)wp & 15) == 0) {
                const f32x4 c0 = *(const f32x4 DION_GLOBAL*)wp, c1 = *(const f32x4 DION_GLOBAL*)(wp + 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  cur[i] = c0[i];
                  cur[4 + i] = c1[i];
                }
              } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) cur[i] = gj0 + i < cols_valid ? wp[i] : 0.f;
              }
            } else {
              const uint16_t DION_GLOBAL* wp = to_global((const uint16_t*)d.out) + o;
              if (full && ((uintptr_t)wp & 15) == 0) {
                const u32x4 b = *(const u32x4 DION_GLOBAL*)wp;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  cur[2 * i] = __uint_as_float(b[i] << 16);
                  cur[2 * i + 1] = __uint_as_float(b[i] & 0xFFFF0000u);
                }
              } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                  cur[i] = gj0 + i < cols_valid ? __uint_as_float((uint32_t)wp[i] << 16) : 0.f;
              }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
              w[i] = __fsub_rn(__fmul_rn(cur[i], pa.upd_keep), __fmul_rn(d.upd_alpha, w[i]));
          }
          if (pa.out_fp32) {
            float DION_GLOBAL* out = to_global_w((float*)d.out) + o;
            if (full && ((uintptr_t)out & 15) == 0) {
              *(f32x4 DION_GLOBAL*)out = f32x4{w[0], w[1], w[2], w[3]};
              *(f32x4 DION_GLOBAL*)(out + 4) = f32x4{w[4], w[5], w[6], w[7]};
            } else {
#pragma unroll
              for (int i = 0; i < 8; ++i)
                if (gj0 + i < cols_valid) out[i] = w[i];
            }
          } else if (pa.out_f16) {
            _Float16 DION_GLOBAL* out = to_global_w((_Float16*)d.out) + o;
            if (full && ((uintptr_t)out & 15) == 0) {
              half8v pk;
#pragma unroll
              for (int i = 0; i < 8; ++i) pk[i] = (_Float16)w[i];
              *(half8v DION_GLOBAL*)out = pk;
            } else {
#pragma unroll
              for (int i = 0; i < 8; ++i)
                if (gj0 + i < cols_valid) out[i] = (_Float16)w[i];
            }
          } else {
            uint16_t DION_GLOBAL* out = to_global_w((uint16_t*)d.out) + o;
            if (full && ((uintptr_t)out & 15) == 0) {
              u32x4 pk;
              pk[0] = (uint32_t)f32_to_bf16_rne(w[0]) | ((uint32_t)f32_to_bf16_rne(w[1]) << 16);
              pk[1] = (uint32_t)f32_to_bf16_rne(w[2]) | ((uint32_t)f32_to_bf16_rne(w[3]) << 16);
              pk[2] = (uint32_t)f32_to_bf16_rne(w[4]) | ((uint32_t)f32_to_bf16_rne(w[5]) << 16);
              pk[3] = (uint32_t)f32_to_bf16_rne(w[6]) | ((uint32_t)f32_to_bf16_rne(w[7]) << 16);
              *(u32x4 DION_GLOBAL*)out = pk;
            } else {
#pragma unroll
              for (int i = 0; i < 8; ++i)
                if (gj0 + i < cols_valid) out[i] = f32_to_bf16_rne(w[i]);
            }
          }
        }
      } else {  // EPI_SYM, EPI_POLY, EPI_RECT, EPI_RECT_T
        store8_split(C, cts, cld, gi, gj0, w, 0xFFu, pa.out_lo != 0);
      }
    }
    wave_lds_sync();

    if (TRANS) {
      // ---- transposed copy from registers.  Lane (c, h) = (lane % 32, lane / 32)
      // holds rows gi0 + 8q + 4h + (0..3) of column gj, i.e. columns
      // 8q + 4h + (0..3) of transposed row gj.  Targets: the mirror C[gj][gi]
      // of a symmetric tile, or the hi term of X = (X^T)^T into aux (ld =
      // arows).  The mirror leaves as 8-byte stores.  For X, lanes c and c + 32
      // first swap halves so that each lane holds whole 8-column chunks (q even
      // in lane h = 0, q odd in lane h = 1), and a pair of chunks leaves as one
      // instruction writing 32 contiguous bytes per row (chunk pairs stay
      // adjacent under the panel swizzle); measured on one box, the exchange
      // gains 2% on the restart apply and loses 2% on the mirrored products.
      _Float16* T = EPI == EPI_RECT_T ? (_Float16*)d.buf[pa.aux_slot] : C;
      const int tld = EPI == EPI_RECT_T ? arows : cld;
      const bool tlo = EPI != EPI_RECT_T && pa.out_lo != 0;
      _Float16 DION_GLOBAL* g = to_global_w(T);
      if constexpr (EPI == EPI_RECT_T) {
        const int h = lane >> 5;
#pragma unroll
        for (int b = 0; b < F; ++b) {
          const int gj = col_base + b * 32 + (lane & 31);
#pragma unroll
          for (int qp = 0; qp < 4; qp += 2) {
            uint32_t hw[2][2];   // own values of chunks qp and qp + 1, as fp16 pairs
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
              for (int i = 0; i < 2; ++i) {
                const _Float16 h0 = (_Float16)v[b][(qp + u) * 4 + 2 * i];
                const _Float16 h1 = (_Float16)v[b][(qp + u) * 4 + 2 * i + 1];
                hw[u][i] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
              }
            // lane h = 0 keeps chunk qp and sends its half of chunk qp + 1;
            // lane h = 1 keeps chunk qp + 1 and sends its half of chunk qp
            uint32_t rh[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) rh[i] = (uint32_t)__shfl_xor((int)hw[1 - h][i], 32, 64);
            // h = 0 owns the low half of its chunk, h = 1 the high half
            const u32x4 ch = h == 0 ? u32x4{hw[0][0], hw[0][1], rh[0], rh[1]}
                                    : u32x4{rh[0], rh[1], hw[1][0], hw[1][1]};
            const int gi0 = row_base + a * 32 + (qp + h) * 8;   // chunk start (a multiple of 8)
            *(u32x4 DION_GLOBAL*)(g + blk_off(gj, gi0, tld)) = ch;
          }
        }
      } else {
#pragma unroll
        for (int b = 0; b < F; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int gj = col_base + b * 32 + (lane & 31);
            const int gi0 = row_base + a * 32 + q * 8 + (lane >> 5) * 4;
            half4 hh, ll;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float x = v[b][q * 4 + i];
              hh[i] = (_Float16)x;
              ll[i] = (_Float16)(x - (float)hh[i]);
            }
            const size_t off = blk_off(gj, gi0, tld);   // 4 contiguous elements (gi0 % 4 == 0)
            *(half4 DION_GLOBAL*)(g + off) = hh;
            if (tlo) *(half4 DION_GLOBAL*)(g + off + cts) = ll;
          }
      }
    }
  }
}

template <int BM, int EPI, int F, int... As>
__device__ __forceinline__ void epilogue_all(const MatDesc& d, const PhaseArgs& pa, float alpha, int arows,
                                             int brows, int ti, int tj, int wm, int wn, int lane,
                                             const floatx16 (&acc)[F][F], float* st,
                                             std::integer_sequence<int, As...>) {
  // the tile's position is uniform over the block: diagonal tiles of
  // symmetric outputs take the variant without the mirror
  if ((EPI == EPI_SYM || EPI == EPI_POLY) && ti == tj)
    (epilogue_strip<BM, EPI, F, As, true>(d, pa, alpha, arows, brows, ti, tj, wm, wn, lane, acc, st), ...);
  else
    (epilogue_strip<BM, EPI, F, As, false>(d, pa, alpha, arows, brows, ti, tj, wm, wn, lane, acc, st), ...);
}

template <int BM, int EPI, int F>
__device__ __forceinline__ void epilogue_strips(const MatDesc& d, const PhaseArgs& pa, int mi, int arows,
                                                int brows, int ti, int tj, int wm, int wn, int lane,
                                                const floatx16 (&acc)[F][F], float* st) {
  const float alpha = phase_alpha<float>(d, pa, mi);
  epilogue_all<BM, EPI, F>(d, pa, alpha, arows, brows, ti, tj, wm, wn, lane, acc, st,
                           std::make_integer_sequence<int, F>{});
}

// ------------------------------------------------------- MFMA16 GEMM kernel
// Global -> LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4,
// scalar base + 32-bit per-lane byte offset): lane l of the wave writes LDS
// bytes [lds + 16 l, lds + 16 l + 16).  Issued through asm so that the
// compiler does not turn every barrier into a wait for all copies in flight;
// completion is tracked by the explicit vmcnt waits of the pipeline.
__device__ __forceinline__ void dma16s(uint32_t voff, const void* sbase, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" : : : "memory"); }
__device__ __forceinline__ const void* sgpr_ptr(const void* p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

// products of the term pairs kept: (0,0), then (0,1) and (1,0) for two-term operands
template <int NA, int NB> struct Prods {
  static constexpr int n = (NA == 2 && NB == 2) ? 3 : ((NA == 2 || NB == 2) ? 2 : 1);
  static constexpr int sa(int p) { return (NA == 2 && NB == 2) ? (p == 2 ? 1 : 0) : (NA == 2 ? p : 0); }
  static constexpr int sb(int p) { return (NA == 2 && NB == 2) ? (p == 1 ? 1 : 0) : (NB == 2 ? p : 0); }
};

// 256 threads = 4 waves in a 2 x 2 grid; each wave owns a (BM/2) x (BM/2)
// sub-tile made of 32 x 32 MFMA blocks.  The K loop is an S-stage pipeline of
// LDS buffers filled by direct global -> LDS copies S - 1 stages ahead, one
// barrier per stage.  A stage holds BK = 32 columns of every operand term;
// each stage row is 64 bytes of 16-byte chunks whose order is XOR-swizzled by
// the row so that the 16-byte fragment reads of 8 or 16 lanes hit distinct
// banks.  The operands are stored panel-blocked with that swizzle applied
// (blk_off), so one term of one stage is a single contiguous run of whole
// cache lines that each lane copies 16 bytes of, linearly.  Within a stage the
// two 16-deep halves are software-pipelined through two register sets, and
// every LDS fragment read and every copy is issued right after an MFMA, so
// that the matrix pipe stays fed while they go out: the MFMAs of half 1 of
// stage k-1 carry the reads of half 0 of stage k, the MFMAs of half 0 of
// stage k carry the reads of half 1, and the copies of stage k+S-1 ride in
// between, one per two MFMAs over both halves.
template <int BM, int NA, int NB, int EPI, bool SYM>
__global__ __launch_bounds__(256, (BM == 128 && NA + NB == 2) ? 3 : 1) void k_gemm16(const MatDesc* __restrict__ descs,
                                                   const int* __restrict__ mats,
                                                   const int* __restrict__ prefix, int nmat,
                                                   const int* __restrict__ ranges, PhaseArgs pa) {
  constexpr int NT = NA + NB;
  constexpr int BK = 32;
  constexpr int SLOTS = BK / 8;              // 16-byte chunks per stage row
  constexpr int RPW = 128 / BK;              // stage rows per 256-byte bank window
  constexpr int TERM_BYTES = BM * BK * 2;    // one operand term of one stage
  constexpr int STAGE_BYTES = NT * TERM_BYTES;
  constexpr int S = (BM == 128 && NT == 2) ? 3
                  : (4 * STAGE_BYTES <= 160 * 1024 ? 4 : (3 * STAGE_BYTES <= 160 * 1024 ? 3 : 2));
  constexpr int IPW = TERM_BYTES / 4096;     // 1 KB copies per wave per term per stage
  constexpr int WT = BM / 2;                 // wave tile
  constexpr int F = WT / 32;                 // MFMA blocks per wave dim
  constexpr int NMF = Prods<NA, NB>::n * F * F;  // MFMAs per half-stage
  constexpr int NRD = NT * F;                // fragment reads per half-stage
  constexpr int NDMA = IPW * NT;             // copies per stage per wave
  constexpr int MAIN_BYTES = S * STAGE_BYTES;
  constexpr int EPI_BYTES = 4 * epi_wave_bytes(WT);
  constexpr int LDS_BYTES = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;
  static_assert(IPW >= 1 && S >= 2, "tile too small for the copy layout");
  static_assert(NDMA % 2 == 0 && NDMA / 2 <= NMF / 2 && NRD <= NMF,
                "every fragment read and copy needs an MFMA slot");
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

  const int t = range_tile(ranges, blockIdx.x);
  if (t < 0) return;
  const int j = find_segment(prefix, nmat, t);
  const int mi = mats[j];
  const MatDesc& d = descs[mi];
  const int arows = pa.a_rows_is_n ? d.n_pad : d.m_pad;
  const int brows = pa.b_rows_is_n ? d.n_pad : d.m_pad;
  const int K = pa.k_is_n ? d.n_pad : d.m_pad;
  int ti, tj;
  decode_tile(SYM, t - prefix[j], arows, brows, BM, ti, tj);

  // panel-blocked operands: the tile's rows start inside row-block (ti*BM)/256;
  // stage kt is column-block kt, 16 KB further on per block (8 KB per tile
  // when BM = 128, which covers half of the block's rows)
  const char* gA = (const char*)((const _Float16*)d.buf[pa.a_slot] + blk_off(ti * BM, 0, K));
  const char* gB = (const char*)((const _Float16*)d.buf[pa.b_slot] + blk_off(tj * BM, 0, K));
  const size_t a_ts = (size_t)arows * K * 2, b_ts = (size_t)brows * K * 2;   // term strides, bytes

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)smem);

  // per-lane byte offsets of the copies: a stage of one term is a contiguous
  // TERM_BYTES run of the blocked operand, copied linearly (same for A and B)
  uint32_t voff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) voff[i] = (uint32_t)((i * 4 + wave) * 1024 + lane * 16);
  // q-th copy of the stage held in LDS buffer st, K columns from k0
  auto dma = [&](int q, int st, int k0) {
    const int i = q / NT, u = q % NT;
    const char* base = u < NA ? gA + u * a_ts : gB + (u - NA) * b_ts;
    dma16s(voff[i], sgpr_ptr(base + (size_t)(k0 >> 5) * 16384),
           (uint32_t)__builtin_amdgcn_readfirstlane(lds0 + st * STAGE_BYTES + (i * 4 + wave) * 1024 + u * TERM_BYTES));
  };

  floatx16 acc[F][F];
#pragma unroll
  for (int a = 0; a < F; ++a)
#pragma unroll
    for (int b = 0; b < F; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  // per-lane LDS element offsets of the fragments (f = 0; +32 rows per f)
  const int rowa = wm * WT + (lane & 31), rowb = wn * WT + (lane & 31);
  const int swa = (rowa / RPW) & (SLOTS - 1), swb = (rowb / RPW) & (SLOTS - 1);
  int offa[2], offb[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int chunk = kk * 2 + (lane >> 5);
    offa[kk] = rowa * BK + ((chunk ^ swa) << 3);
    offb[kk] = rowb * BK + ((chunk ^ swb) << 3);
  }
  half8 fa[2][NA][F], fb[2][NB][F];   // two register sets of one half-stage's fragments
  // q-th fragment read of half kk of the stage at sb into register set r
  auto rd = [&](int q, const _Float16* sb, int kk, int r) {
    if (q < NA * F) {
      const int u = q / F, f = q % F;
      fa[r][u][f] = *(const half8*)(sb + u * (TERM_BYTES / 2) + offa[kk] + f * 32 * BK);
    } else {
      const int q2 = q - NA * F, u = q2 / F, f = q2 % F;
      fb[r][u][f] = *(const half8*)(sb + (NA + u) * (TERM_BYTES / 2) + offb[kk] + f * 32 * BK);
    }
  };
  auto mf = [&](int q, int r) {
    const int p = q / (F * F), a = (q / F) % F, b = q % F;
    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[r][Prods<NA, NB>::sa(p)][a], fb[r][Prods<NA, NB>::sb(p)][b],
                                                       acc[a][b], 0, 0, 0);
  };

  const int nk = K / BK;   // >= 8: every dimension is padded to a multiple of 256
  const int klast = (nk - 1) * BK;
#pragma unroll
  for (int st = 0; st < S - 1; ++st)
#pragma unroll
    for (int q = 0; q < NDMA; ++q) dma(q, st, st * BK);

  // stage 0: wait, then read half 0 (set 0) and issue the copies of stage S-1
  wait_vmcnt<(S - 2) * NDMA>();
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
  {
    const _Float16* sb = (const _Float16*)smem;
#pragma unroll
    for (int q = 0; q < NRD; ++q) rd(q, sb, 0, 0);
#pragma unroll
    for (int q = 0; q < NDMA; ++q) dma(q, (S - 1) % S, min((S - 1) * BK, klast));
    __builtin_amdgcn_sched_barrier(0);
    // MFMAs of half 0 (set 0) carry the reads of half 1 into set 1
#pragma unroll
    for (int q = 0; q < NMF; ++q) {
      mf(q, 0);
      if (q < NRD) rd(q, sb, 1, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  for (int kt = 1; kt < nk; ++kt) {
    wait_lgkm0();                     // this wave's reads of stage kt-1 are done
    wait_vmcnt<(S - 2) * NDMA>();     // this wave's copies of stage kt have landed
    lds_barrier();                    // ... and every wave's
    __builtin_amdgcn_sched_barrier(0);
    const _Float16* sb = (const _Float16*)(smem + (kt % S) * STAGE_BYTES);
    const int st_next = (kt + S - 1) % S;
    const int k_next = min((kt + S - 1) * BK, klast);   // past the end: a harmless re-copy
    // Each half's MFMAs carry that half's fragment reads in even slots and
    // half of the copies of stage kt+S-1 in odd slots, so copies leave at one
    // per two MFMAs over the whole stage.  Copies of the second half may go
    // out too: their buffer held stage kt-1, read and consumed by every wave
    // before the barrier.
    auto slot = [&](int q, int half, int r_set) {
      if (q % 2 == 0 && q / 2 < NRD) rd(q / 2, sb, half, r_set);
      if (q % 2 == 1) {
        if (q / 2 < NDMA / 2) dma(half * (NDMA / 2) + q / 2, st_next, k_next);
        if (NRD > NMF / 2 && q / 2 + NMF / 2 < NRD) rd(q / 2 + NMF / 2, sb, half, r_set);
      }
    };
    // half 1 of stage kt-1 (set 1) carries the reads of half 0 of stage kt (set 0)
#pragma unroll
    for (int q = 0; q < NMF; ++q) {
      mf(q, 1);
      slot(q, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // half 0 of stage kt (set 0) carries the reads of half 1 of stage kt (set 1)
#pragma unroll
    for (int q = 0; q < NMF; ++q) {
      mf(q, 0);
      slot(q, 1, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int q = 0; q < NMF; ++q) mf(q, 1);

  // epilogue: acc[a][b][e] holds C[row][col] of the wave's sub-tile with
  //   row = a*32 + (e/4)*8 + (lane/32)*4 + e%4,  col = b*32 + lane%32
  wait_vmcnt<0>();    // the re-copies past the end land before LDS is reused
  __syncthreads();
  epilogue_strips<BM, EPI, F>(d, pa, mi, arows, brows, ti, tj, wm, wn, lane, acc,
                              (float*)smem + wave * (epi_wave_bytes(WT) / 4));
}

// --------------------------------------------------------- FP64 GEMM kernel
// 64 x 64 tiles, 256 threads as 16 x 16, each thread a 4 x 4 block; BK = 16.
template <int EPI, bool SYM>
__global__ __launch_bounds__(256) void k_gemm64(const MatDesc* __restrict__ descs,
                                                const int* __restrict__ mats,
                                                const int* __restrict__ prefix, int nmat,
                                                const int* __restrict__ ranges, PhaseArgs pa) {
  constexpr int BM = 64, BK = 16;
  __shared__ double sA[BK][BM + 1];
  __shared__ double sB[BK][BM + 1];
  const int t = range_tile(ranges, blockIdx.x);
  if (t < 0) return;
  const int j = find_segment(prefix, nmat, t);
  const int mi = mats[j];
  const MatDesc& d = descs[mi];
  const int arows = pa.a_rows_is_n ? d.n_pad : d.m_pad;
  const int brows = pa.b_rows_is_n ? d.n_pad : d.m_pad;
  const int K = pa.k_is_n ? d.n_pad : d.m_pad;
  int ti, tj;
  decode_tile(SYM, t - prefix[j], arows, brows, BM, ti, tj);
  const double DION_GLOBAL* gA = to_global((const double*)d.buf[pa.a_slot]) + (size_t)ti * BM * K;
  const double DION_GLOBAL* gB = to_global((const double*)d.buf[pa.b_slot]) + (size_t)tj * BM * K;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  double acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    // 64 rows x 16 k per operand = 1024 values, 4 per thread
    for (int q = 0; q < 4; ++q) {
      const int v = threadIdx.x + 256 * q;
      const int row = v >> 4, kk = v & 15;
      sA[kk][row] = gA[(size_t)row * K + k0 + kk];
      sB[kk][row] = gB[(size_t)row * K + k0 + kk];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      double a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = sA[kk][ty * 4 + i]; b[i] = sB[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = fma(a[i], b[jj], acc[i][jj]);
    }
    __syncthreads();
  }
  const double alpha = phase_alpha<double>(d, pa, mi);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      epilogue_elem<EPI, double, double>(d, pa, arows, brows, ti, tj, BM, ty * 4 + i, tx * 4 + jj,
                                         acc[i][jj], alpha);
}

// ---------------------------------------------------------------- launchers
#define DION_G16(BM_, NA_, NB_, EPI_, SYM_) \
  hipLaunchKernelGGL((k_gemm16<BM_, NA_, NB_, EPI_, SYM_>), dim3(grid), dim3(256), 0, stream, \
                     L.descs, L.mats, L.prefix, L.nmat, L.ranges, pa)

// Returns false for an unsupported combination.
bool launch_gemm16(int bm, int na, int nb, int epi, bool sym, const GemmLaunch& L,
                   const PhaseArgs& pa, hipStream_t stream) {
  if (L.total <= 0) return true;
  const int grid = L.grid;
  const int key = (na << 8) | (nb << 4) | epi;
#define DION_CASES(BM_)                                                                  \
  if (sym) {                                                                             \
    switch (key) {                                                                       \
      case (1 << 8) | (1 << 4) | EPI_SYM: DION_G16(BM_, 1, 1, EPI_SYM, true); return true; \
      case (2 << 8) | (2 << 4) | EPI_SYM: DION_G16(BM_, 2, 2, EPI_SYM, true); return true; \
      case (2 << 8) | (2 << 4) | EPI_POLY: DION_G16(BM_, 2, 2, EPI_POLY, true); return true; \
      case (1 << 8) | (1 << 4) | EPI_POLY: DION_G16(BM_, 1, 1, EPI_POLY, true); return true; \
      default: return false;                                                             \
    }                                                                                    \
  } else {                                                                               \
    switch (key) {                                                                       \
      case (1 << 8) | (1 << 4) | EPI_RECT: DION_G16(BM_, 1, 1, EPI_RECT, false); return true; \
      case (2 << 8) | (1 << 4) | EPI_RECT: DION_G16(BM_, 2, 1, EPI_RECT, false); return true; \
      case (1 << 8) | (1 << 4) | EPI_RECT_T: DION_G16(BM_, 1, 1, EPI_RECT_T, false); return true; \
      case (2 << 8) | (1 << 4) | EPI_RECT_T: DION_G16(BM_, 2, 1, EPI_RECT_T, false); return true; \
      case (1 << 8) | (1 << 4) | EPI_OUT: DION_G16(BM_, 1, 1, EPI_OUT, false); return true; \
      case (2 << 8) | (1 << 4) | EPI_OUT: DION_G16(BM_, 2, 1, EPI_OUT, false); return true; \
      case (1 << 8) | (2 << 4) | EPI_OUT: DION_G16(BM_, 1, 2, EPI_OUT, false); return true; \
      case (2 << 8) | (2 << 4) | EPI_OUT: DION_G16(BM_, 2, 2, EPI_OUT, false); return true; \
      default: return false;                                                             \
    }                                                                                    \
  }
  if (bm == 256) { DION_CASES(256) }
  else if (bm == 128) { DION_CASES(128) }
  return false;
#undef DION_CASES
}
#undef DION_G16

bool launch_gemm64(int epi, bool sym, const GemmLaunch& L, const PhaseArgs& pa, hipStream_t stream) {
  if (L.total <= 0) return true;
  const int grid = L.grid;
#define DION_G64(EPI_, SYM_) \
  hipLaunchKernelGGL((k_gemm64<EPI_, SYM_>), dim3(grid), dim3(256), 0, stream, L.descs, L.mats, \
                     L.prefix, L.nmat, L.ranges, pa)
  if (sym) {
    if (epi == EPI_SYM) { DION_G64(EPI_SYM, true); return true; }
    if (epi == EPI_POLY) { DION_G64(EPI_POLY, true); return true; }
  } else {
    if (epi == EPI_RECT) { DION_G64(EPI_RECT, false); return true; }
    if (epi == EPI_OUT) { DION_G64(EPI_OUT, false); return true; }
  }
  return false;
#undef DION_G64
}

}  // namespace dion
