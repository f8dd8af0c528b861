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
#include <cstring>
#include <type_traits>

#include "dion_internal.h"

namespace dion {

// Global-address-space pointers (vmcnt only; flat accesses also count
// against the LDS wait counter) and native vector types for them.
#define DION_SGLOBAL __attribute__((address_space(1)))
typedef uint32_t pk_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t pk_u32x4 __attribute__((ext_vector_type(4)));
typedef float pk_f32x4 __attribute__((ext_vector_type(4)));

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
// A row's key is the exact sum of the squares of its stored values, rounded
// once to the nearest double (ties to even).  A correctly rounded sum does not
// depend on the order of summation, so the rows it selects are the ones any
// implementation that rounds the exact sum once selects.  The square of a
// float32 value (bf16 and fp16 values included) is exact in fp64.
//
// Fast path: each lane keeps its running sum as an unevaluated pair hi + lo,
// updated by two error-free additions (Knuth's TwoSum), and raises a flag when
// the second addition rounds; the wave combines the lanes' pairs the same
// way.  Without the flag hi + lo is the exact sum and one IEEE addition
// fl(hi + lo) rounds it correctly.  The flag needs the squares of a row to
// spread over more than about 106 bits (a value near 2^-45 times the row's
// largest).  Then the wave reads the row again and adds the squares into an
// exact 640-bit fixed-point integer per lane, whose unit 2^-298 is the
// weight of the smallest square; the lanes' integers are summed and the total
// is rounded once.  Rows with an Inf or NaN get a NaN key.
//
// 16-bit inputs take a cheaper fast path.  The square of a value with p
// significant bits (8 for bf16, 11 for fp16) is an integer multiple of
// 2^(2 E - 254 - 2 (p - 1)), E its exponent in fp32 (at least 1), so every
// square in a group of a lane's values, and every partial sum of them, is a
// multiple of 2^L with L taken at the group's smallest nonzero exponent.  A
// multiple of 2^L below 2^(L + 53) is a double, so the group's plain fp64 sum
// is exact as long as its partial sums stay below that bound; they only
// grow, and rounding is monotone, so the final sum is below the bound exactly
// when none of them crossed it.  A group is the eight values of one 16-byte
// load: it costs one fused multiply-add and one integer minimum per value,
// and its exact sum enters the TwoSum pair as one term.  A group whose sum
// reaches the bound (its squares spread over more than about 2^34 for bf16,
// 2^28 for fp16: one value in some 10^5 of a Gaussian row) or is Inf or NaN
// adds its values to the pair one at a time instead.  (Groups of 64 values
// send too many rows to the integer fallback: a bf16 value 10^-5 times the
// scale of its group is enough.)
//
// At row_frac = 1 no row is chosen by its key: the keys only give ||M||_F^2,
// and the plain fp64 sum (EXACT = false) serves.

__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = __dadd_rn(a, b);
  const double bb = __dsub_rn(s, a);
  e = __dadd_rn(__dsub_rn(a, __dsub_rn(s, bb)), __dsub_rn(b, bb));
}

struct SqAcc {
  double hi = 0.0, lo = 0.0;
  unsigned bad = 0u;
  __device__ __forceinline__ void add(float x) {
    add_exact(__dmul_rn((double)x, (double)x));         // exact: 48 significant bits at most
  }
  __device__ __forceinline__ void add_exact(double q) {
    double s, e, t, f;
    two_sum(hi, q, s, e);
    two_sum(lo, e, t, f);
    hi = s;
    lo = t;
    bad |= f != 0.0 ? 1u : 0u;
  }
  // afterwards every lane holds the wave's pair and flag (both partners of an
  // exchange form the same sums: TwoSum's result does not depend on the order)
  __device__ __forceinline__ void wave() {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double h2 = __shfl_xor(hi, o, 64), l2 = __shfl_xor(lo, o, 64);
      const unsigned b2 = __shfl_xor(bad, o, 64);
      double s, e, t, f1, u, f2;
      two_sum(hi, h2, s, e);
      two_sum(lo, l2, t, f1);
      two_sum(t, e, u, f2);
      hi = s;
      lo = u;
      bad |= b2 | (f1 != 0.0 ? 1u : 0u) | (f2 != 0.0 ? 1u : 0u);
    }
  }
};

constexpr int SQ_WORDS = 20;   // 640 bits: squares reach 2^256, 2^31 of them fit

// The exact fallback.  Each lane adds its squares into its own 640-bit
// integer in LDS (lane-private words, so the word index may differ between
// lanes).  The wave then sums the integers column by column (lane j < 20 adds
// word j of all 64 lanes) and propagates the carries, leaving word j of the
// total in lane j; the rounding reads the words it needs with shuffles and
// ballots, so no lane ever holds the whole integer.
struct SqExact {
  uint32_t* base;              // the wave's 64 x SQ_WORDS words in LDS
  int lane;
  unsigned special = 0u;       // an Inf or NaN was seen
  uint32_t word = 0u;          // after wave(): word `lane` of the total (lanes < SQ_WORDS)
  __device__ __forceinline__ SqExact(uint32_t* wave_words, int lane_) : base(wave_words), lane(lane_) {
    uint32_t* a = base + lane * SQ_WORDS;
    for (int j = 0; j < SQ_WORDS; ++j) a[j] = 0u;
  }
  // x = m 2^(E - 150) (E >= 1) or f 2^-149 (E = 0), so x^2 = m^2 2^(pos - 298)
  // with m^2 < 2^48 and pos = 2E - 2 (0 for E = 0): pos <= 508, so the three
  // words from pos / 32 stay below word 18
  __device__ __forceinline__ void add(float x) {
    uint32_t* a = base + lane * SQ_WORDS;
    const uint32_t u = __float_as_uint(x);
    const uint32_t E = (u >> 23) & 0xFFu, f = u & 0x7FFFFFu;
    special |= E == 0xFFu ? 1u : 0u;
    const uint64_t m = E ? (uint64_t)(f | 0x800000u) : (uint64_t)f;
    const int pos = E ? 2 * (int)E - 2 : 0;
    const uint64_t v = m * m;
    const int wi = pos >> 5, sh = pos & 31;
    const uint64_t lo = v << sh;
    uint64_t t = (uint64_t)a[wi] + (uint32_t)lo;
    a[wi] = (uint32_t)t;
    t = (uint64_t)a[wi + 1] + (uint32_t)(lo >> 32) + (t >> 32);
    a[wi + 1] = (uint32_t)t;
    t = (uint64_t)a[wi + 2] + (sh ? (uint32_t)(v >> (64 - sh)) : 0u) + (t >> 32);
    a[wi + 2] = (uint32_t)t;
    uint32_t carry = (uint32_t)(t >> 32);
    for (int j = wi + 3; carry && j < SQ_WORDS; ++j) {
      t = (uint64_t)a[j] + carry;
      a[j] = (uint32_t)t;
      carry = (uint32_t)(t >> 32);
    }
  }
  __device__ __forceinline__ void wave() {
    // every lane's words are written before any lane reads another's
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint64_t col = 0;   // at most 64 (2^32 - 1) < 2^38
    if (lane < SQ_WORDS)
      for (int l = 0; l < 64; ++l) col += base[l * SQ_WORDS + lane];
    uint64_t carry = 0;
    for (int j = 0; j < SQ_WORDS; ++j) {
      const uint64_t t = __shfl(col, j, 64) + carry;
      if (lane == j) word = (uint32_t)t;
      carry = t >> 32;
    }
    special = __any(special) ? 1u : 0u;
  }
  __device__ __forceinline__ uint32_t word_at(int j) const {   // j wave-uniform, >= 0
    const uint32_t v = __shfl(word, j < SQ_WORDS ? j : 0, 64);
    return j < SQ_WORDS ? v : 0u;
  }
  // bits [lo, lo + 64) of the total, lo >= 0 and wave-uniform
  __device__ __forceinline__ uint64_t bits(int lo) const {
    const int wi = lo >> 5, sh = lo & 31;
    const uint64_t pq = ((uint64_t)word_at(wi + 1) << 32) | word_at(wi);
    return sh ? (pq >> sh) | ((uint64_t)word_at(wi + 2) << (64 - sh)) : pq;
  }
  // the total times 2^-298, rounded to the nearest double, ties to even
  __device__ __forceinline__ double rounded() const {
    if (special) return __longlong_as_double(0x7FF8000000000000ll);
    const unsigned long long nz = __ballot(lane < SQ_WORDS && word != 0u);
    if (!nz) return 0.0;
    const int tw = 63 - __clzll((long long)nz);                // highest nonzero word
    const int top = 32 * tw + 31 - __clz((int)word_at(tw));    // highest set bit
    if (top <= 52) return ldexp((double)bits(0), -298);       // 53 bits at most: exact
    int ex = top - 52;                                         // weight of the last kept bit
    uint64_t mant = bits(ex) & ((1ull << 53) - 1ull);
    const int g = ex - 1;                                      // guard bit
    const unsigned guard = (unsigned)(bits(g) & 1ull);
    // sticky: any bit below the guard bit, from the words each lane holds
    const int b0 = 32 * lane;
    const uint32_t mask = b0 + 32 <= g ? 0xFFFFFFFFu : (b0 >= g ? 0u : ((1u << (g - b0)) - 1u));
    const bool sticky = __ballot(lane < SQ_WORDS && (word & mask) != 0u) != 0ull;
    if (guard && (sticky || (mant & 1ull))) ++mant;
    if (mant >> 53) {   // rounded up into the next binade
      mant >>= 1;
      ++ex;
    }
    return ldexp((double)mant, ex - 298);
  }
};
// LDS words of the fallback: one 640-bit integer per lane of a 256-thread block (20 KB)
constexpr int SQ_LDS_WORDS = 256 * SQ_WORDS;

// Calls f(x) on the elements of row r that this lane owns: 8 consecutive
// 16-bit or 4 consecutive fp32 values per lane and step when the row allows
// 16-byte loads, else one element per lane and step.
template <typename InT, typename F>
__device__ __forceinline__ void row_elems(const MatDesc& d, int64_t r, int lane, F&& f) {
  const InT* row = (const InT*)d.M + r * d.C;
  if (sizeof(InT) == 2) {
    const uint16_t* p = (const uint16_t*)row;
    if ((d.C & 7) == 0 && ((uintptr_t)d.M & 15) == 0) {
      for (int c = lane * 8; c < d.C; c += 512) {
        const uint4 v = *(const uint4*)(p + c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f(in16_to_f32<InT>(w[q] & 0xFFFFu));
          f(in16_to_f32<InT>(w[q] >> 16));
        }
      }
    } else {
      for (int c = lane; c < d.C; c += 64) f(in16_to_f32<InT>(p[c]));
    }
  } else {
    const float* p = (const float*)row;
    if ((d.C & 3) == 0 && ((uintptr_t)d.M & 15) == 0) {
      for (int c = lane * 4; c < d.C; c += 256) {
        const float4 v = *(const float4*)(p + c);
        f(v.x);
        f(v.y);
        f(v.z);
        f(v.w);
      }
    } else {
      for (int c = lane; c < d.C; c += 64) f(p[c]);
    }
  }
}

// One wave per row.
template <typename InT, bool EXACT>
__global__ __launch_bounds__(256) void k_rowkeys(const MatDesc* __restrict__ descs, int nmat,
                                                 int64_t total_rows, double* __restrict__ keys) {
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (g >= total_rows) return;
  const MatDesc& d = descs[mat_of_row(descs, nmat, g)];
  const int64_t r = g - d.row0;
  double key;
  if (!EXACT) {
    double s = 0.0;
    row_elems<InT>(d, r, lane, [&](float x) { s += (double)x * (double)x; });
    key = wave_sum(s);
  } else {
    SqAcc A;
    const bool vec16 = sizeof(InT) == 2 && (d.C & 7) == 0 && ((uintptr_t)d.M & 15) == 0;
    if (vec16) {
      constexpr int p = std::is_same<InT, _Float16>::value ? 11 : 8;   // significant bits
      const uint16_t* row = (const uint16_t*)d.M + r * d.C;
      for (int c = lane * 8; c < d.C; c += 512) {
        const uint4 v = *(const uint4*)(row + c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float xs[8];
        double s = 0.0;
        uint32_t amin = 0xFFFFFFFFu;     // of (fp32 bits << 1) - 1: sign dropped, zeros wrap to the top
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          xs[q] = in16_to_f32<InT>(q & 1 ? w[q >> 1] >> 16 : w[q >> 1] & 0xFFFFu);
          s = __fma_rn((double)xs[q], (double)xs[q], s);
          amin = min(amin, (__float_as_uint(xs[q]) << 1) - 1u);
        }
        if (amin != 0xFFFFFFFFu) {
          const int E = max((int)((amin + 1u) >> 24), 1);
          const int L = 2 * E - 254 - 2 * (p - 1);
          const double bound = __longlong_as_double((long long)(L + 53 + 1023) << 52);   // 2^(L + 53)
          if (s < bound) {               // false for Inf and NaN too
            A.add_exact(s);
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) A.add(xs[q]);
          }
        }
      }
    } else {
      row_elems<InT>(d, r, lane, [&](float x) { A.add(x); });
    }
    A.wave();
    if (!A.bad) {
      key = __dadd_rn(A.hi, A.lo);
    } else {   // wave-uniform: every lane holds the combined flag
      __shared__ uint32_t sq_lds[SQ_LDS_WORDS];
      SqExact X(sq_lds + (threadIdx.x & ~63u) * SQ_WORDS, lane);
      const InT* row = (const InT*)d.M + r * d.C;
#pragma unroll 1
      for (int c = lane; c < d.C; c += 64) {
        float x;
        if (sizeof(InT) == 2) x = in16_to_f32<InT>(((const uint16_t*)row)[c]);
        else x = ((const float*)row)[c];
        X.add(x);
      }
      X.wave();
      key = X.rounded();
    }
  }
  if (lane == 0) keys[g] = key;
}

// ---------------------------------------------- momentum / error feedback
// E <- fl32(fl32(beta * E) + grad), key <- the key of the new row of E (as
// above), and out <- bf16(E) (write_out 1), out <- 0 (write_out 2: the carry
// form of error feedback, where unselected rows contribute no update) or
// nothing (write_out 0: out is the weight of the fused update).  __fmul_rn /
// __fadd_rn keep the two roundings separate (no contraction); beta = 1 gives
// fl32(E + grad).  The exact fallback reads the new E back with the same
// lane-to-element map as the pass that wrote it, so each lane reads its own
// stores.
template <typename GT, bool EXACT>
__global__ __launch_bounds__(256) void k_momentum_keys(const MatDesc* __restrict__ descs, int nmat,
                                                       int64_t total_rows, float beta,
                                                       double* __restrict__ keys, int write_out) {
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (g >= total_rows) return;
  const MatDesc& d = descs[mat_of_row(descs, nmat, g)];
  const int64_t r = g - d.row0;
  // global-address-space accesses: flat ones would also count against the
  // LDS wait counter, so the row's closing reduction would wait for its stores
  float DION_SGLOBAL* E = (float DION_SGLOBAL*)d.M + r * d.C;
  uint16_t DION_SGLOBAL* out = (uint16_t DION_SGLOBAL*)d.out + r * d.C;
  const uint16_t DION_SGLOBAL* G16 = (const uint16_t DION_SGLOBAL*)d.grad + r * d.C;
  const float DION_SGLOBAL* G32 = (const float DION_SGLOBAL*)d.grad + r * d.C;
  double s = 0.0;
  SqAcc A;
  auto key_of = [&](float m) {
    if (EXACT) A.add(m);
    else s += (double)m * (double)m;
  };
  const bool vec = (d.C & 3) == 0;
  if (vec) {
    // every byte is touched once: non-temporal loads and stores (2-3% on the
    // Llama-3-8B layer set's pass, paired runs on one box)
    for (int c = lane * 4; c < d.C; c += 256) {
      const pk_f32x4 e = __builtin_nontemporal_load((const pk_f32x4 DION_SGLOBAL*)(E + c));
      float gv[4];
      if (sizeof(GT) == 2) {
        const pk_u32x2 b = __builtin_nontemporal_load((const pk_u32x2 DION_SGLOBAL*)(G16 + c));
        gv[0] = __uint_as_float(b[0] << 16);
        gv[1] = __uint_as_float(b[0] & 0xFFFF0000u);
        gv[2] = __uint_as_float(b[1] << 16);
        gv[3] = __uint_as_float(b[1] & 0xFFFF0000u);
      } else {
        const pk_f32x4 b = __builtin_nontemporal_load((const pk_f32x4 DION_SGLOBAL*)(G32 + c));
        gv[0] = b[0]; gv[1] = b[1]; gv[2] = b[2]; gv[3] = b[3];
      }
      float m[4] = {__fadd_rn(__fmul_rn(beta, e[0]), gv[0]), __fadd_rn(__fmul_rn(beta, e[1]), gv[1]),
                    __fadd_rn(__fmul_rn(beta, e[2]), gv[2]), __fadd_rn(__fmul_rn(beta, e[3]), gv[3])};
      __builtin_nontemporal_store(pk_f32x4{m[0], m[1], m[2], m[3]}, (pk_f32x4 DION_SGLOBAL*)(E + c));
      if (write_out == 1) {
        const pk_u32x2 o = {(uint32_t)bf16_rne(m[0]) | ((uint32_t)bf16_rne(m[1]) << 16),
                            (uint32_t)bf16_rne(m[2]) | ((uint32_t)bf16_rne(m[3]) << 16)};
        __builtin_nontemporal_store(o, (pk_u32x2 DION_SGLOBAL*)(out + c));
      } else if (write_out == 2) {
        *(pk_u32x2 DION_SGLOBAL*)(out + c) = pk_u32x2{0u, 0u};
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) key_of(m[q]);
    }
  } else {
    for (int c = lane; c < d.C; c += 64) {
      const float gv = sizeof(GT) == 2 ? bf16_to_f32(G16[c]) : G32[c];
      const float m = __fadd_rn(__fmul_rn(beta, E[c]), gv);
      E[c] = m;
      if (write_out) out[c] = write_out == 1 ? bf16_rne(m) : (uint16_t)0;
      key_of(m);
    }
  }
  double key;
  if (!EXACT) {
    key = wave_sum(s);
  } else {
    A.wave();
    if (!A.bad) {
      key = __dadd_rn(A.hi, A.lo);
    } else {
      __shared__ uint32_t sq_lds[SQ_LDS_WORDS];
      SqExact X(sq_lds + (threadIdx.x & ~63u) * SQ_WORDS, lane);
      if (vec) {
#pragma unroll 1
        for (int c = lane * 4; c < d.C; c += 256)
#pragma unroll 1
          for (int q = 0; q < 4; ++q) X.add(E[c + q]);
      } else {
#pragma unroll 1
        for (int c = lane; c < d.C; c += 64) X.add(E[c]);
      }
      X.wave();
      key = X.rounded();
    }
  }
  if (lane == 0) keys[g] = key;
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
__global__ __launch_bounds__(256) void k_pack(const MatDesc* __restrict__ descs, const int* __restrict__ mats,
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
  const MatDesc& d = descs[mats[lo]];
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
__global__ __launch_bounds__(256) void k_pack16(const MatDesc* __restrict__ descs, const int* __restrict__ mats,
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
  const int mi = mats[lo];
  const MatDesc& d = descs[mi];
  const int local = t - prefix[lo];
  const int k_pad = d.tall ? d.n_pad : d.m_pad;
  const int c_pad = d.tall ? d.m_pad : d.n_pad;
  const int tc = c_pad / 64;
  const int r0 = (local / tc) * 64, c0 = (local % tc) * 64;
  const float scale = ldexpf(1.0f, scalars[mi].e);
  const int* idx = idx_all + d.sel0;
  _Float16* sl = (_Float16*)(d.tall ? d.buf[SLOT_XT0] : d.buf[SLOT_X]);
  _Float16* st = (_Float16*)(d.tall ? d.buf[SLOT_X] : d.buf[SLOT_XT0]);
  const bool sl_lo = d.tall && xterms > 1, st_lo = !d.tall && xterms > 1;
  const size_t ts = (size_t)k_pad * c_pad;
  const bool vec = (d.C & 7) == 0 && ((uintptr_t)d.M & 15) == 0;

  // loads and stores through global pointers (flat ones would also count
  // against the LDS wait counter), and every store after the barrier, so
  // that neither the barrier nor an LDS wait waits for a store
  auto split_store = [&](_Float16* base, size_t off, const float* v, bool with_lo) {
    half8s h, l;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h[i] = (_Float16)v[i];
      l[i] = (_Float16)(v[i] - (float)h[i]);
    }
    _Float16 DION_SGLOBAL* g = (_Float16 DION_SGLOBAL*)base + off;
    *(half8s DION_SGLOBAL*)g = h;
    if (with_lo) *(half8s DION_SGLOBAL*)(g + ts) = l;
  };
  float v[2][8];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = threadIdx.x + 256 * j;
    const int row = q >> 3, cc = (q & 7) * 8;
    const int r = r0 + row, c = c0 + cc;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[j][i] = 0.f;
    if (r < d.k && c < d.C) {
      const int src = use_idx ? ((const int DION_SGLOBAL*)idx)[r] : r;
      const InT DION_SGLOBAL* p = (const InT DION_SGLOBAL*)d.M + (int64_t)src * d.C + c;
      if (vec) {  // c + 8 <= C: C and c are multiples of 8
        if (sizeof(InT) == 2) {
          const pk_u32x4 u = *(const pk_u32x4 DION_SGLOBAL*)p;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[j][2 * i] = in16_to_f32<InT>(u[i] & 0xFFFFu);
            v[j][2 * i + 1] = in16_to_f32<InT>(u[i] >> 16);
          }
        } else {
          const pk_f32x4 a = ((const pk_f32x4 DION_SGLOBAL*)p)[0], b = ((const pk_f32x4 DION_SGLOBAL*)p)[1];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[j][i] = a[i];
            v[j][4 + i] = b[i];
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (c + i < d.C)
            v[j][i] = sizeof(InT) == 2 ? in16_to_f32<InT>(((const uint16_t DION_SGLOBAL*)p)[i])
                                       : ((const float DION_SGLOBAL*)p)[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[j][i] *= scale;
      tile[row][cc + i] = v[j][i];
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = threadIdx.x + 256 * j;
    const int row = q >> 3, cc = (q & 7) * 8;
    split_store(sl, blk_off(r0 + row, c0 + cc, c_pad), v[j], sl_lo);   // SL row r, columns c..c+7
  }
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
__global__ __launch_bounds__(256) void k_transpose(const MatDesc* __restrict__ descs, const int* __restrict__ mats,
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
  const MatDesc& d = descs[mats[lo]];
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
  // global-address-space pointers and non-temporal accesses: every byte is
  // touched once
  const float DION_SGLOBAL* E = (const float DION_SGLOBAL*)d.M + r * d.C;
  uint16_t DION_SGLOBAL* W16 = (uint16_t DION_SGLOBAL*)d.out + r * d.C;
  float DION_SGLOBAL* W32 = (float DION_SGLOBAL*)d.out + r * d.C;
  const float al = d.upd_alpha;
  if ((d.C & 3) == 0) {   // 4 consecutive elements per lane (rows start 16-byte aligned)
    for (int c = lane * 4; c < d.C; c += 256) {
      const pk_f32x4 e = __builtin_nontemporal_load((const pk_f32x4 DION_SGLOBAL*)(E + c));
      float wv[4];
      if (sizeof(WT) == 2) {
        const pk_u32x2 b = __builtin_nontemporal_load((const pk_u32x2 DION_SGLOBAL*)(W16 + c));
        wv[0] = __uint_as_float(b[0] << 16);
        wv[1] = __uint_as_float(b[0] & 0xFFFF0000u);
        wv[2] = __uint_as_float(b[1] << 16);
        wv[3] = __uint_as_float(b[1] & 0xFFFF0000u);
      } else {
        const pk_f32x4 b = __builtin_nontemporal_load((const pk_f32x4 DION_SGLOBAL*)(W32 + c));
        wv[0] = b[0]; wv[1] = b[1]; wv[2] = b[2]; wv[3] = b[3];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        wv[q] = raw ? __fsub_rn(__fmul_rn(wv[q], keep), __fmul_rn(al, e[q])) : __fmul_rn(wv[q], keep);
      if (sizeof(WT) == 2) {
        const pk_u32x2 o = {(uint32_t)bf16_rne(wv[0]) | ((uint32_t)bf16_rne(wv[1]) << 16),
                            (uint32_t)bf16_rne(wv[2]) | ((uint32_t)bf16_rne(wv[3]) << 16)};
        __builtin_nontemporal_store(o, (pk_u32x2 DION_SGLOBAL*)(W16 + c));
      } else {
        __builtin_nontemporal_store(pk_f32x4{wv[0], wv[1], wv[2], wv[3]}, (pk_f32x4 DION_SGLOBAL*)(W32 + c));
      }
    }
  } else {
    for (int c = lane; c < d.C; c += 64) {
      const float w = sizeof(WT) == 2 ? bf16_to_f32(W16[c]) : W32[c];
      const float v = raw ? __fsub_rn(__fmul_rn(w, keep), __fmul_rn(al, E[c])) : __fmul_rn(w, keep);
      if (sizeof(WT) == 2) W16[c] = bf16_rne(v);
      else W32[c] = v;
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

// ------------------------------------------------- plan upload by value
// The allocation-free entry point has no pinned staging buffer: the plan
// header travels to the device as kernel arguments, 2 KB per launch, and a
// copy kernel stores it.  The arguments are copied at launch, so the host
// blob may be reused at once.
constexpr int UPLOAD_WORDS = 512;
struct UploadChunk {
  uint32_t w[UPLOAD_WORDS];
};

__global__ __launch_bounds__(256) void k_upload(uint32_t* __restrict__ dst, UploadChunk c, int nwords) {
  for (int i = threadIdx.x; i < nwords; i += 256) dst[i] = c.w[i];
}

// ---------------------------------------------------------------- launchers
static inline unsigned row_blocks(int64_t rows) { return (unsigned)((rows + 3) / 4); }

// fmt: the storage format of the inputs, 0 = bf16, 1 = fp32, 2 = fp16
void launch_rowkeys(int fmt, bool exact, const MatDesc* descs, int nmat, int64_t rows, double* keys,
                    hipStream_t s) {
#define DION_KEYS(T_, X_) hipLaunchKernelGGL((k_rowkeys<T_, X_>), dim3(row_blocks(rows)), dim3(256), 0, s, descs, nmat, rows, keys)
  if (exact) {
    if (fmt == 0) DION_KEYS(uint16_t, true);
    else if (fmt == 2) DION_KEYS(_Float16, true);
    else DION_KEYS(float, true);
  } else {
    if (fmt == 0) DION_KEYS(uint16_t, false);
    else if (fmt == 2) DION_KEYS(_Float16, false);
    else DION_KEYS(float, false);
  }
#undef DION_KEYS
}

void launch_momentum_keys(bool grad_bf16, bool exact, const MatDesc* descs, int nmat, int64_t rows, float beta,
                          double* keys, int write_out, hipStream_t s) {
#define DION_MOM(T_, X_) hipLaunchKernelGGL((k_momentum_keys<T_, X_>), dim3(row_blocks(rows)), dim3(256), 0, s, descs, nmat, rows, beta, keys, write_out)
  if (exact) {
    if (grad_bf16) DION_MOM(uint16_t, true);
    else DION_MOM(float, true);
  } else {
    if (grad_bf16) DION_MOM(uint16_t, false);
    else DION_MOM(float, false);
  }
#undef DION_MOM
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

void launch_pack(int fmt, bool fp64_path, const MatDesc* descs, const int* mats, const int* prefix, int nmat,
                 int total, const int* idx, const MatScalars* scalars, int xterms, bool use_idx,
                 hipStream_t s) {
  if (total <= 0) return;
  const int ui = use_idx ? 1 : 0;
#define DION_PACK(K_, T_) hipLaunchKernelGGL((K_<T_>), dim3(total), dim3(256), 0, s, descs, mats, prefix, nmat, total, idx, scalars, xterms, ui)
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

void launch_transpose(const MatDesc* descs, const int* mats, const int* prefix, int nmat, int total, int src_slot,
                      int dst_slot, hipStream_t s) {
  if (total <= 0) return;
  hipLaunchKernelGGL(k_transpose<double>, dim3(total), dim3(256), 0, s, descs, mats, prefix, nmat, total, src_slot,
                     dst_slot);
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

// bytes: a multiple of 4; src: host memory, read before this returns
void launch_upload(void* dst, const void* src, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  for (size_t w0 = 0; w0 < words; w0 += UPLOAD_WORDS) {
    UploadChunk c;
    const int n = (int)(words - w0 < (size_t)UPLOAD_WORDS ? words - w0 : (size_t)UPLOAD_WORDS);
    memcpy(c.w, (const uint32_t*)src + w0, 4 * (size_t)n);
    hipLaunchKernelGGL(k_upload, dim3(1), dim3(256), 0, s, (uint32_t*)dst + w0, c, n);
  }
}

void launch_scale_combine(MatScalars* scalars, int nmat, hipStream_t s) {
  hipLaunchKernelGGL(k_scale_combine, dim3((nmat + 255) / 256), dim3(256), 0, s, scalars, nmat);
}

}  // namespace dion
