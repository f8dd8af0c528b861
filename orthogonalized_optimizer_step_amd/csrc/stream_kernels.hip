// HBM-bound passes around the MFMA phases: row keys, the fp32 momentum /
// error-feedback update, top-k row selection with the Frobenius norm,
// gather + convert + transpose into the padded operand buffers, transposes,
// and the copy of unselected rows.
//
// Row rule: the Dion3 abstract and the Dion3 summary (方法 / 核心模块, "Dion3
// 更新规则" bullet) select a fraction of the momentum rows each step; the
// pages name no criterion, so rows are ranked by squared L2 norm (fp64, from
// the exact stored values), larger first, ties to the lower row index.
// Momentum: the summary's flow (输入输出流程) updates the momentum first; the
// fp32 buffer is updated by two separately rounded fp32 operations.
#include "dion_internal.h"

namespace dion {

__device__ __forceinline__ uint16_t bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// 16-bit input element -> fp32: InT = uint16_t holds bf16 bits, _Float16 holds fp16.
template <typename InT> __device__ __forceinline__ float in16_to_f32(uint32_t b);
template <> __device__ __forceinline__ float in16_to_f32<uint16_t>(uint32_t b) { return bf16_to_f32((uint16_t)b); }
template <> __device__ __forceinline__ float in16_to_f32<_Float16>(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
template <> __device__ __forceinline__ float in16_to_f32<float>(uint32_t b) { return __uint_as_float(b); }  // unused

__device__ __forceinline__ double wave_sum(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// global row -> matrix (descs are in batch order with increasing row0)
__device__ __forceinline__ int mat_of_row(const MatDesc* descs, int nmat, int64_t g) {
  int lo = 0, hi = nmat;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (descs[mid].row0 <= g) lo = mid; else hi = mid;
  }
  return lo;
}

// ------------------------------------------------------------ row keys
// One wave per row: key = sum_c x^2 in fp64 (each square is exact in fp64).
template <typename InT>
__global__ __launch_bounds__(256) void k_rowkeys(const MatDesc* __restrict__ descs, int nmat,
                                                 int64_t total_rows, double* __restrict__ keys) {
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (g >= total_rows) return;
  const MatDesc& d = descs[mat_of_row(descs, nmat, g)];
  const int64_t r = g - d.row0;
  const InT* row = (const InT*)d.M + r * d.C;
  double s = 0.0;
  if (sizeof(InT) == 2) {
    const uint16_t* p = (const uint16_t*)row;
    if ((d.C & 7) == 0) {
      for (int c = lane * 8; c < d.C; c += 512) {
        uint4 v = *(const uint4*)(p + c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const double lo = (double)in16_to_f32<InT>(w[q] & 0xFFFFu);
          const double hi = (double)in16_to_f32<InT>(w[q] >> 16);
          s += lo * lo;
          s += hi * hi;
        }
      }
    } else {
      for (int c = lane; c < d.C; c += 64) {
        const double x = (double)in16_to_f32<InT>(p[c]);
        s += x * x;
      }
    }
  } else {
    const float* p = (const float*)row;
    if ((d.C & 3) == 0) {
      for (int c = lane * 4; c < d.C; c += 256) {
        float4 v = *(const float4*)(p + c);
        s += (double)v.x * v.x;
        s += (double)v.y * v.y;
        s += (double)v.z * v.z;
        s += (double)v.w * v.w;
      }
    } else {
      for (int c = lane; c < d.C; c += 64) {
        const double x = (double)p[c];
        s += x * x;
      }
    }
  }
  s = wave_sum(s);
  if (lane == 0) keys[g] = s;
}

// ---------------------------------------------- momentum / error feedback
// E <- fl32(fl32(beta * E) + grad), key <- sum E^2 (fp64), and out <- bf16(E)
// (write_out 1), out <- 0 (write_out 2: the carry form of error feedback,
// where unselected rows contribute no update) or nothing (write_out 0: out is
// the weight of the fused update).  __fmul_rn / __fadd_rn keep the two
// roundings separate (no contraction); beta = 1 gives fl32(E + grad).
template <typename GT>
__global__ __launch_bounds__(256) void k_momentum_keys(const MatDesc* __restrict__ descs, int nmat,
                                                       int64_t total_rows, float beta,
                                                       double* __restrict__ keys, int write_out) {
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (g >= total_rows) return;
  const MatDesc& d = descs[mat_of_row(descs, nmat, g)];
  const int64_t r = g - d.row0;
  float* E = (float*)d.M + r * d.C;
  uint16_t* out = (uint16_t*)d.out + r * d.C;
  double s = 0.0;
  if ((d.C & 3) == 0) {
    for (int c = lane * 4; c < d.C; c += 256) {
      float4 e = *(float4*)(E + c);
      float gv[4];
      if (sizeof(GT) == 2) {
        const uint2 b = *(const uint2*)((const uint16_t*)d.grad + r * d.C + c);
        gv[0] = __uint_as_float(b.x << 16);
        gv[1] = __uint_as_float(b.x & 0xFFFF0000u);
        gv[2] = __uint_as_float(b.y << 16);
        gv[3] = __uint_as_float(b.y & 0xFFFF0000u);
      } else {
        const float4 b = *(const float4*)((const float*)d.grad + r * d.C + c);
        gv[0] = b.x; gv[1] = b.y; gv[2] = b.z; gv[3] = b.w;
      }
      float m[4] = {__fadd_rn(__fmul_rn(beta, e.x), gv[0]), __fadd_rn(__fmul_rn(beta, e.y), gv[1]),
                    __fadd_rn(__fmul_rn(beta, e.z), gv[2]), __fadd_rn(__fmul_rn(beta, e.w), gv[3])};
      *(float4*)(E + c) = make_float4(m[0], m[1], m[2], m[3]);
      if (write_out == 1) {
        uint2 o;
        o.x = (uint32_t)bf16_rne(m[0]) | ((uint32_t)bf16_rne(m[1]) << 16);
        o.y = (uint32_t)bf16_rne(m[2]) | ((uint32_t)bf16_rne(m[3]) << 16);
        *(uint2*)(out + c) = o;
      } else if (write_out == 2) {
        *(uint2*)(out + c) = make_uint2(0u, 0u);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) s += (double)m[q] * (double)m[q];
    }
  } else {
    for (int c = lane; c < d.C; c += 64) {
      const float gv = sizeof(GT) == 2 ? bf16_to_f32(((const uint16_t*)d.grad)[r * d.C + c])
                                       : ((const float*)d.grad)[r * d.C + c];
      const float m = __fadd_rn(__fmul_rn(beta, E[c]), gv);
      E[c] = m;
      if (write_out) out[c] = write_out == 1 ? bf16_rne(m) : (uint16_t)0;
      s += (double)m * (double)m;
    }
  }
  s = wave_sum(s);
  if (lane == 0) keys[g] = s;
}

// ------------------------------------------------- selection + norm
// One 1024-thread block per matrix.  Top-k by (key desc, row asc): an MSB
// first radix select over the 64-bit key patterns (non-negative doubles order
// like their bit patterns) finds the k-th largest key T and how many rows
// equal to T are needed; ranks among equal keys and the ascending compaction
// come from block scans in row order.  The squared Frobenius norm of the
// selected rows is the sum of their keys, reduced in a fixed order.
constexpr int SEL_THREADS = 1024;

__device__ int block_excl_scan(int v, int* sh, int& total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int o = 1; o < SEL_THREADS; o <<= 1) {
    const int add = tid >= o ? sh[tid - o] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  const int incl = sh[tid];
  total = sh[SEL_THREADS - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(SEL_THREADS) void k_select(const MatDesc* __restrict__ descs,
                                                        const double* __restrict__ keys_all,
                                                        uint8_t* __restrict__ flags_all,
                                                        int* __restrict__ idx_all,
                                                        MatScalars* __restrict__ scalars,
                                                        int fp64_path) {
  __shared__ unsigned hist[256];
  __shared__ int scan_sh[SEL_THREADS];
  __shared__ double red[SEL_THREADS];
  __shared__ int s_digit, s_need;
  const MatDesc& d = descs[blockIdx.x];
  const int R = d.R, k = d.k, tid = threadIdx.x;
  const double* keys = keys_all + d.row0;
  uint8_t* flags = flags_all + d.row0;
  int* idx = idx_all + d.sel0;
  const uint64_t* ukeys = (const uint64_t*)keys;

  uint64_t T = 0;
  int need = 0;  // rows with key == T still to take
  if (k < R) {
    uint64_t prefix = 0, mask = 0;
    int kk = k;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += SEL_THREADS) hist[i] = 0;
      __syncthreads();
      for (int r = tid; r < R; r += SEL_THREADS) {
        const uint64_t u = ukeys[r];
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int cum = 0, dg = 0;
        for (dg = 255; dg >= 0; --dg) {
          if (cum + (int)hist[dg] >= kk) break;
          cum += hist[dg];
        }
        s_digit = dg < 0 ? 0 : dg;
        s_need = kk - cum;
      }
      __syncthreads();
      prefix |= (uint64_t)s_digit << shift;
      mask |= (uint64_t)0xFF << shift;
      kk = s_need;
      __syncthreads();
    }
    T = prefix;
    need = kk;
  }

  // flags + ascending compaction, chunk by chunk in row order
  int eq_base = 0, sel_base = 0;
  for (int base = 0; base < R; base += SEL_THREADS) {
    const int r = base + tid;
    const bool valid = r < R;
    int sel = 0;
    if (k >= R) {
      sel = valid;
    } else {
      const uint64_t u = valid ? ukeys[r] : 0;
      const int is_eq = valid && u == T;
      int tot;
      const int rank = block_excl_scan(is_eq, scan_sh, tot);
      sel = valid && (u > T || (is_eq && eq_base + rank < need));
      eq_base += tot;
    }
    int tot2;
    const int pos = block_excl_scan(sel, scan_sh, tot2);
    if (valid) flags[r] = (uint8_t)sel;
    if (sel && sel_base + pos < k) idx[sel_base + pos] = r;
    sel_base += tot2;
  }
  __syncthreads();

  // squared Frobenius norm of the selected rows, fixed-order reduction
  double s = 0.0;
  for (int r = tid; r < R; r += SEL_THREADS)
    if (flags[r]) s += keys[r];
  red[tid] = s;
  __syncthreads();
  for (int o = SEL_THREADS / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) {
    const double nu2 = red[0];
    MatScalars sc;
    sc.nu2 = nu2;
    if (nu2 > 0.0) {
      const double nu = sqrt(nu2);
      int E2;
      frexp(nu, &E2);  // nu <= 2^E2
      const int e = fp64_path ? 0 : 14 - E2;  // |S * 2^e| <= nu 2^(14-E2) <= 2^14
      sc.e = e;
      sc.x0_alpha64 = ldexp(1.0, -e) / nu;
    } else {
      sc.e = 0;
      sc.x0_alpha64 = 0.0;
    }
    sc.x0_alpha = (float)sc.x0_alpha64;
    scalars[blockIdx.x] = sc;
  }
}

// ------------------------------------------------------------- pack
// S = M[selected rows] (k x C) into the padded operand buffers:
//   SL [k_pad][C_pad] (S as is) and ST [C_pad][k_pad] (S transposed).
// wide (k <= C): X = SL, X^T = ST;  tall: X = ST, X^T = SL.
// The Gram operand X keeps one term; X^T keeps `xterms` terms (hi, lo).
// MFMA16 values are S * 2^e rounded to fp16 (exact for bf16 input within
// fp16's normal range), panel-blocked; FP64 values are S exactly, row-major.
// 64 x 64 tiles via LDS.

// FP64 path.
template <typename InT>
__global__ __launch_bounds__(256) void k_pack(const MatDesc* __restrict__ descs,
                                              const int* __restrict__ prefix, int nmat, int total,
                                              const int* __restrict__ idx_all,
                                              const MatScalars* __restrict__ scalars, int xterms,
                                              int use_idx) {
  __shared__ float tile[64][65];
  const int t = blockIdx.x;
  if (t >= total) return;
  int lo = 0, hi = nmat;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (prefix[mid] <= t) lo = mid; else hi = mid;
  }
  const MatDesc& d = descs[lo];
  const int local = t - prefix[lo];
  const int k_pad = d.tall ? d.n_pad : d.m_pad;
  const int c_pad = d.tall ? d.m_pad : d.n_pad;
  const int tc = c_pad / 64;
  const int r0 = (local / tc) * 64, c0 = (local % tc) * 64;
  const int* idx = idx_all + d.sel0;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;

  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    float v = 0.f;
    if (r < d.k && c < d.C) {
      const int src = use_idx ? idx[r] : r;
      const InT* row = (const InT*)d.M + (int64_t)src * d.C;
      if (sizeof(InT) == 2) v = in16_to_f32<InT>(((const uint16_t*)row)[c]);
      else v = ((const float*)row)[c];
    }
    tile[i][tx] = v;
  }
  __syncthreads();
  double* sl = (double*)(d.tall ? d.buf[SLOT_XT0] : d.buf[SLOT_X]);
  double* st = (double*)(d.tall ? d.buf[SLOT_X] : d.buf[SLOT_XT0]);
  for (int i = ty; i < 64; i += 4) {
    sl[(size_t)(r0 + i) * c_pad + c0 + tx] = (double)tile[i][tx];   // SL row r0+i, column c0+tx
    st[(size_t)(c0 + i) * k_pad + r0 + tx] = (double)tile[tx][i];   // ST row c0+i, column r0+tx
  }
}

// MFMA16 path: 16-byte row loads (when rows are 16-byte aligned), SL stored
// as 8-column chunks straight from registers, ST through a 64 x 65 fp32 LDS
// tile read as 8-row column chunks (both LDS passes are bank-conflict-free).
typedef _Float16 half8s __attribute__((ext_vector_type(8)));
template <typename InT>
__global__ __launch_bounds__(256) void k_pack16(const MatDesc* __restrict__ descs,
                                                const int* __restrict__ prefix, int nmat, int total,
                                                const int* __restrict__ idx_all,
                                                const MatScalars* __restrict__ scalars, int xterms,
                                                int use_idx) {
  __shared__ float tile[64][65];
  const int t = blockIdx.x;
  if (t >= total) return;
  int lo = 0, hi = nmat;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (prefix[mid] <= t) lo = mid; else hi = mid;
  }
  const MatDesc& d = descs[lo];
  const int local = t - prefix[lo];
  const int k_pad = d.tall ? d.n_pad : d.m_pad;
  const int c_pad = d.tall ? d.m_pad : d.n_pad;
  const int tc = c_pad / 64;
  const int r0 = (local / tc) * 64, c0 = (local % tc) * 64;
  const float scale = ldexpf(1.0f, scalars[lo].e);
  const int* idx = idx_all + d.sel0;
  _Float16* sl = (_Float16*)(d.tall ? d.buf[SLOT_XT0] : d.buf[SLOT_X]);
  _Float16* st = (_Float16*)(d.tall ? d.buf[SLOT_X] : d.buf[SLOT_XT0]);
  const bool sl_lo = d.tall && xterms > 1, st_lo = !d.tall && xterms > 1;
  const size_t ts = (size_t)k_pad * c_pad;
  const bool vec = (d.C & 7) == 0 && ((uintptr_t)d.M & 15) == 0;

  auto split_store = [&](_Float16* base, size_t off, const float* v, bool with_lo) {
    half8s h, l;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h[i] = (_Float16)v[i];
      l[i] = (_Float16)(v[i] - (float)h[i]);
    }
    *(half8s*)(base + off) = h;
    if (with_lo) *(half8s*)(base + off + ts) = l;
  };
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = threadIdx.x + 256 * j;
    const int row = q >> 3, cc = (q & 7) * 8;
    const int r = r0 + row, c = c0 + cc;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
    if (r < d.k && c < d.C) {
      const int src = use_idx ? idx[r] : r;
      const InT* p = (const InT*)d.M + (int64_t)src * d.C + c;
      if (vec) {  // c + 8 <= C: C and c are multiples of 8
        if (sizeof(InT) == 2) {
          const uint4 u = *(const uint4*)p;
          const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[2 * i] = in16_to_f32<InT>(w4[i] & 0xFFFFu);
            v[2 * i + 1] = in16_to_f32<InT>(w4[i] >> 16);
          }
        } else {
          const float4 a = ((const float4*)p)[0], b = ((const float4*)p)[1];
          v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
          v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (c + i < d.C)
            v[i] = sizeof(InT) == 2 ? in16_to_f32<InT>(((const uint16_t*)p)[i]) : ((const float*)p)[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] *= scale;
      tile[row][cc + i] = v[i];
    }
    split_store(sl, blk_off(r, c, c_pad), v, sl_lo);      // SL row r, columns c..c+7
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = threadIdx.x + 256 * j;
    const int col = q >> 3, rr = (q & 7) * 8;
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = tile[rr + i][col];
    split_store(st, blk_off(c0 + col, r0 + rr, k_pad), w, st_lo);   // ST row c0+col, columns r0+rr..+7
  }
}

// ---------------------------------------------------------- transpose
// FP64 path: X^T [n_pad][m_pad] -> X [m_pad][n_pad], row-major (the MFMA16 path
// writes X in the restart apply's epilogue).
template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const MatDesc* __restrict__ descs,
                                                   const int* __restrict__ prefix, int nmat,
                                                   int total, int src_slot, int dst_slot) {
  __shared__ T tile[64][65];
  const int t = blockIdx.x;
  if (t >= total) return;
  int lo = 0, hi = nmat;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (prefix[mid] <= t) lo = mid; else hi = mid;
  }
  const MatDesc& d = descs[lo];
  const int local = t - prefix[lo];
  const int tm = d.m_pad / 64;
  const int n0 = (local / tm) * 64, m0 = (local % tm) * 64;
  const T* src = (const T*)d.buf[src_slot];
  T* dst = (T*)d.buf[dst_slot];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) tile[i][tx] = src[(size_t)(n0 + i) * d.m_pad + m0 + tx];
  __syncthreads();
  for (int i = ty; i < 64; i += 4) dst[(size_t)(m0 + i) * d.n_pad + n0 + tx] = tile[tx][i];
}

// ------------------------------------------------- unselected row copy
template <typename InT>
__global__ __launch_bounds__(256) void k_copy_unselected(const MatDesc* __restrict__ descs, int nmat,
                                                         int64_t total_rows,
                                                         const uint8_t* __restrict__ flags) {
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (g >= total_rows || flags[g]) return;
  const MatDesc& d = descs[mat_of_row(descs, nmat, g)];
  const int64_t r = g - d.row0;
  const InT* src = (const InT*)d.M + r * d.C;
  InT* dst = (InT*)d.out + r * d.C;
  const size_t bytes = (size_t)d.C * sizeof(InT);
  if (((bytes | (uintptr_t)src | (uintptr_t)dst) & 15) == 0) {
    // 16 bytes per lane, two chunks in flight per lane
    const uint4* s4 = (const uint4*)src;
    uint4* d4 = (uint4*)dst;
    const int n = (int)(bytes >> 4);
    int c = lane;
    for (; c + 64 < n; c += 128) {
      const uint4 x0 = s4[c], x1 = s4[c + 64];
      d4[c] = x0;
      d4[c + 64] = x1;
    }
    if (c < n) d4[c] = s4[c];
  } else {
    for (int c = lane; c < d.C; c += 64) dst[c] = src[c];
  }
}

// ------------------------------------------- weight update, unselected rows
// Fused weight update of a row-subset step: the rows the selection left out
// carry the raw momentum E (fp32, already updated), so
// W <- fl32(fl32(W * keep) - fl32(alpha * E)), rounded to W's dtype.  One wave
// per row; selected rows are left to the final apply's epilogue.
template <typename WT>
__global__ __launch_bounds__(256) void k_update_unselected(const MatDesc* __restrict__ descs, int nmat,
                                                           int64_t total_rows, const uint8_t* __restrict__ flags,
                                                           float keep, int raw) {
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (g >= total_rows || flags[g]) return;
  const MatDesc& d = descs[mat_of_row(descs, nmat, g)];
  const int64_t r = g - d.row0;
  const float* E = (const float*)d.M + r * d.C;
  WT* W = (WT*)d.out + r * d.C;
  const float al = d.upd_alpha;
  if ((d.C & 3) == 0) {   // 4 consecutive elements per lane (rows start 16-byte aligned)
    for (int c = lane * 4; c < d.C; c += 256) {
      const float4 e = *(const float4*)(E + c);
      const float ev[4] = {e.x, e.y, e.z, e.w};
      float wv[4];
      if (sizeof(WT) == 2) {
        const uint2 b = *(const uint2*)((const uint16_t*)W + c);
        wv[0] = __uint_as_float(b.x << 16);
        wv[1] = __uint_as_float(b.x & 0xFFFF0000u);
        wv[2] = __uint_as_float(b.y << 16);
        wv[3] = __uint_as_float(b.y & 0xFFFF0000u);
      } else {
        const float4 b = *(const float4*)((const float*)W + c);
        wv[0] = b.x; wv[1] = b.y; wv[2] = b.z; wv[3] = b.w;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        wv[q] = raw ? __fsub_rn(__fmul_rn(wv[q], keep), __fmul_rn(al, ev[q])) : __fmul_rn(wv[q], keep);
      if (sizeof(WT) == 2) {
        uint2 o;
        o.x = (uint32_t)bf16_rne(wv[0]) | ((uint32_t)bf16_rne(wv[1]) << 16);
        o.y = (uint32_t)bf16_rne(wv[2]) | ((uint32_t)bf16_rne(wv[3]) << 16);
        *(uint2*)((uint16_t*)W + c) = o;
      } else {
        *(float4*)((float*)W + c) = make_float4(wv[0], wv[1], wv[2], wv[3]);
      }
    }
  } else {
    for (int c = lane; c < d.C; c += 64) {
      const float w = sizeof(WT) == 2 ? bf16_to_f32(((const uint16_t*)W)[c]) : ((const float*)W)[c];
      const float v = raw ? __fsub_rn(__fmul_rn(w, keep), __fmul_rn(al, E[c])) : __fmul_rn(w, keep);
      if (sizeof(WT) == 2) ((uint16_t*)W)[c] = bf16_rne(v);
      else ((float*)W)[c] = v;
    }
  }
}

// ---------------------------------------- carry: decay of captured rows
// Error feedback in the carry form: after the selected rows of the buffer
// have been packed for orthogonalization, they keep fl32(beta * B); the other
// rows are carried as they are.  One wave per selected row (idx NULL: every
// row is selected).
__global__ __launch_bounds__(256) void k_decay_selected(const MatDesc* __restrict__ descs, int nmat,
                                                        int64_t total_sel, const int* __restrict__ idx,
                                                        float beta) {
  const int64_t s = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (s >= total_sel) return;
  int lo = 0, hi = nmat;   // descs[lo].sel0 <= s < descs[hi].sel0
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (descs[mid].sel0 <= s) lo = mid; else hi = mid;
  }
  const MatDesc& d = descs[lo];
  float* E = (float*)d.M + (idx ? (int64_t)idx[s] : s - d.sel0) * d.C;   // rho = 1: every row
  if ((d.C & 3) == 0) {
    for (int c = lane * 4; c < d.C; c += 256) {
      float4 e = *(float4*)(E + c);
      e.x = __fmul_rn(beta, e.x); e.y = __fmul_rn(beta, e.y); e.z = __fmul_rn(beta, e.z); e.w = __fmul_rn(beta, e.w);
      *(float4*)(E + c) = e;
    }
  } else {
    for (int c = lane; c < d.C; c += 64) E[c] = __fmul_rn(beta, E[c]);
  }
}

// ------------------------------------------------------------ unpack
// Phase entry points: an m x m workspace matrix (slot `slot`; MFMA16: fp16
// hi + lo, panel-blocked; FP64: row-major doubles) -> out (m x m fp32,
// row-major), each value times `scale` (and times the matrix's nu^2 when
// use_nu2).  64 x 64 tiles of the padded matrix; padding is not written.
template <typename ST>
__global__ __launch_bounds__(256) void k_unpack(const MatDesc* __restrict__ descs,
                                                const int* __restrict__ prefix, int nmat, int total,
                                                int slot, const MatScalars* __restrict__ scalars,
                                                float scale, int use_nu2) {
  const int t = blockIdx.x;
  if (t >= total) return;
  int lo = 0, hi = nmat;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (prefix[mid] <= t) lo = mid; else hi = mid;
  }
  const MatDesc& d = descs[lo];
  const int local = t - prefix[lo];
  const int tm = d.m_pad / 64;
  const int r0 = (local / tm) * 64, c0 = (local % tm) * 64;
  const double sc = (double)scale * (use_nu2 ? scalars[lo].nu2 : 1.0);
  float* out = (float*)d.out;
  const size_t ts = (size_t)d.m_pad * d.m_pad;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = r0 + (i >> 6), c = c0 + (i & 63);
    if (r >= d.m || c >= d.m) continue;
    double v;
    if (sizeof(ST) == 8) {
      v = ((const double*)d.buf[slot])[(size_t)r * d.m_pad + c];
    } else {
      const _Float16* b = (const _Float16*)d.buf[slot];
      const size_t o = blk_off(r, c, d.m_pad);
      v = (double)(float)b[o] + (double)(float)b[o + ts];
    }
    out[(size_t)r * d.m + c] = (float)(v * sc);
  }
}

// Phase entry point for the apply: descs [0, nmat) are the X operands and
// [nmat, 2 nmat) the Q operands, each packed as stored * 2^e; the product's
// scale 2^-(e_X + e_Q) goes to the X scalars' x0_alpha.
__global__ void k_scale_combine(MatScalars* __restrict__ scalars, int nmat) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nmat) return;
  const int e = scalars[i].e + scalars[nmat + i].e;
  scalars[i].x0_alpha64 = ldexp(1.0, -e);
  scalars[i].x0_alpha = (float)scalars[i].x0_alpha64;
}

// ---------------------------------------------------------------- launchers
static inline unsigned row_blocks(int64_t rows) { return (unsigned)((rows + 3) / 4); }

// fmt: the storage format of the inputs, 0 = bf16, 1 = fp32, 2 = fp16
void launch_rowkeys(int fmt, const MatDesc* descs, int nmat, int64_t rows, double* keys,
                    hipStream_t s) {
  if (fmt == 0) hipLaunchKernelGGL(k_rowkeys<uint16_t>, dim3(row_blocks(rows)), dim3(256), 0, s, descs, nmat, rows, keys);
  else if (fmt == 2) hipLaunchKernelGGL(k_rowkeys<_Float16>, dim3(row_blocks(rows)), dim3(256), 0, s, descs, nmat, rows, keys);
  else hipLaunchKernelGGL(k_rowkeys<float>, dim3(row_blocks(rows)), dim3(256), 0, s, descs, nmat, rows, keys);
}

void launch_momentum_keys(bool grad_bf16, const MatDesc* descs, int nmat, int64_t rows, float beta,
                          double* keys, int write_out, hipStream_t s) {
  const int wo = write_out;
  if (grad_bf16) hipLaunchKernelGGL(k_momentum_keys<uint16_t>, dim3(row_blocks(rows)), dim3(256), 0, s, descs, nmat, rows, beta, keys, wo);
  else hipLaunchKernelGGL(k_momentum_keys<float>, dim3(row_blocks(rows)), dim3(256), 0, s, descs, nmat, rows, beta, keys, wo);
}

void launch_update_unselected(bool w_bf16, const MatDesc* descs, int nmat, int64_t rows, const uint8_t* flags,
                              float keep, bool raw, hipStream_t s) {
  const int rw = raw ? 1 : 0;
  if (w_bf16) hipLaunchKernelGGL(k_update_unselected<uint16_t>, dim3(row_blocks(rows)), dim3(256), 0, s, descs, nmat, rows, flags, keep, rw);
  else hipLaunchKernelGGL(k_update_unselected<float>, dim3(row_blocks(rows)), dim3(256), 0, s, descs, nmat, rows, flags, keep, rw);
}

void launch_decay_selected(const MatDesc* descs, int nmat, int64_t total_sel, const int* idx, float beta,
                           hipStream_t s) {
  if (total_sel > 0)
    hipLaunchKernelGGL(k_decay_selected, dim3(row_blocks(total_sel)), dim3(256), 0, s, descs, nmat, total_sel, idx, beta);
}

void launch_select(const MatDesc* descs, int nmat, const double* keys, uint8_t* flags, int* idx,
                   MatScalars* scalars, bool fp64_path, hipStream_t s) {
  hipLaunchKernelGGL(k_select, dim3(nmat), dim3(SEL_THREADS), 0, s, descs, keys, flags, idx, scalars,
                     fp64_path ? 1 : 0);
}

void launch_pack(int fmt, bool fp64_path, const MatDesc* descs, const int* prefix, int nmat,
                 int total, const int* idx, const MatScalars* scalars, int xterms, bool use_idx,
                 hipStream_t s) {
  if (total <= 0) return;
  const int ui = use_idx ? 1 : 0;
#define DION_PACK(K_, T_) hipLaunchKernelGGL((K_<T_>), dim3(total), dim3(256), 0, s, descs, prefix, nmat, total, idx, scalars, xterms, ui)
  if (fp64_path) {
    if (fmt == 0) DION_PACK(k_pack, uint16_t);
    else if (fmt == 2) DION_PACK(k_pack, _Float16);
    else DION_PACK(k_pack, float);
  } else {
    if (fmt == 0) DION_PACK(k_pack16, uint16_t);
    else if (fmt == 2) DION_PACK(k_pack16, _Float16);
    else DION_PACK(k_pack16, float);
  }
#undef DION_PACK
}

void launch_transpose(const MatDesc* descs, const int* prefix, int nmat, int total, int src_slot, int dst_slot,
                      hipStream_t s) {
  if (total <= 0) return;
  hipLaunchKernelGGL(k_transpose<double>, dim3(total), dim3(256), 0, s, descs, prefix, nmat, total, src_slot, dst_slot);
}

void launch_copy_unselected(bool bf16, const MatDesc* descs, int nmat, int64_t rows,
                            const uint8_t* flags, hipStream_t s) {
  if (bf16) hipLaunchKernelGGL(k_copy_unselected<uint16_t>, dim3(row_blocks(rows)), dim3(256), 0, s, descs, nmat, rows, flags);
  else hipLaunchKernelGGL(k_copy_unselected<float>, dim3(row_blocks(rows)), dim3(256), 0, s, descs, nmat, rows, flags);
}

void launch_unpack(bool fp64_path, const MatDesc* descs, const int* prefix, int nmat, int total, int slot,
                   const MatScalars* scalars, float scale, bool use_nu2, hipStream_t s) {
  if (total <= 0) return;
  if (fp64_path) hipLaunchKernelGGL(k_unpack<double>, dim3(total), dim3(256), 0, s, descs, prefix, nmat, total, slot, scalars, scale, use_nu2 ? 1 : 0);
  else hipLaunchKernelGGL(k_unpack<_Float16>, dim3(total), dim3(256), 0, s, descs, prefix, nmat, total, slot, scalars, scale, use_nu2 ? 1 : 0);
}

void launch_scale_combine(MatScalars* scalars, int nmat, hipStream_t s) {
  hipLaunchKernelGGL(k_scale_combine, dim3((nmat + 255) / 256), dim3(256), 0, s, scalars, nmat);
}

}  // namespace dion
