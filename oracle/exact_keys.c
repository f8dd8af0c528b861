/*
 * Oracle (test infrastructure only): row keys of the row rule, exactly.
 *
 * The row rule (Dion3 abstract; Dion3 summary, 方法 / 核心模块, "Dion3 更新规则"
 * bullet) keeps a fraction of the momentum rows.  The pages name no
 * criterion; the reading taken is the squared L2 norm of each row.  The key is
 * defined here as the exact sum of the squares of the stored values, rounded
 * once to the nearest double (ties to even): a value that does not depend on
 * any summation order, so every implementation that rounds the exact sum
 * once selects the same rows.
 *
 * Method: plain integer arithmetic.  Every input is a float32 value (bf16 and
 * fp16 values are float32 values too): x = m 2^e with an integer m < 2^24 and
 * e >= -149, so x^2 = m^2 2^(2e) with m^2 < 2^48.  The squares are added into
 * one 640-bit fixed-point integer whose unit is 2^-298 (the smallest square's
 * weight), which holds any sum of up to 2^31 squares without loss.  The
 * integer is then rounded once to 53 significant bits.
 *
 * Shares no code with the HIP library; built with the host C compiler.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define NWORDS 20 /* 32-bit words: 640 bits */

/* acc += v * 2^pos, v < 2^48 */
static void add_shifted(uint32_t* acc, int pos, uint64_t v) {
  int w = pos / 32, sh = pos % 32;
  /* v * 2^sh as three 32-bit pieces */
  uint64_t lo = v << sh;
  uint64_t hi = sh ? v >> (64 - sh) : 0;
  uint32_t piece[3] = {(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi};
  uint64_t carry = 0;
  for (int j = w; j < NWORDS; ++j) {
    uint64_t add = j - w < 3 ? piece[j - w] : 0;
    uint64_t s = (uint64_t)acc[j] + add + carry;
    acc[j] = (uint32_t)s;
    carry = s >> 32;
    if (j - w >= 2 && carry == 0) break;
  }
}

static int bit_at(const uint32_t* acc, int i) { return (int)((acc[i / 32] >> (i % 32)) & 1u); }

/* The integer acc, times 2^-298, rounded to the nearest double (ties to even). */
static double round_to_double(const uint32_t* acc) {
  int top = -1;
  for (int i = 32 * NWORDS - 1; i >= 0; --i)
    if (bit_at(acc, i)) {
      top = i;
      break;
    }
  if (top < 0) return 0.0;
  int lo = top >= 52 ? top - 52 : 0; /* the 53 (or fewer) significant bits */
  uint64_t mant = 0;
  for (int i = top; i >= lo; --i) mant = (mant << 1) | (uint64_t)bit_at(acc, i);
  if (lo > 0) {
    int guard = bit_at(acc, lo - 1), sticky = 0;
    for (int i = lo - 2; i >= 0 && !sticky; --i) sticky = bit_at(acc, i);
    if (guard && (sticky || (mant & 1u))) ++mant;
    if (mant >> 53) { /* rounded up to the next binade */
      mant >>= 1;
      ++lo;
    }
  }
  return ldexp((double)mant, lo - 298);
}

/* keys[r] = the exact sum over c of M[r][c]^2, rounded once to double.
 * M: rows x cols float32, row-major.  Inf or NaN entries give NaN. */
void oracle_row_sumsq_f32(const float* M, int64_t rows, int64_t cols, double* keys) {
  uint32_t acc[NWORDS];
  for (int64_t r = 0; r < rows; ++r) {
    memset(acc, 0, sizeof acc);
    int bad = 0;
    for (int64_t c = 0; c < cols; ++c) {
      uint32_t u;
      memcpy(&u, M + r * cols + c, 4);
      uint32_t E = (u >> 23) & 0xFFu, f = u & 0x7FFFFFu;
      if (E == 0xFFu) {
        bad = 1;
        continue;
      }
      uint64_t m = E ? (f | 0x800000u) : f;
      int e = E ? (int)E - 150 : -149; /* |x| = m 2^e */
      if (m) add_shifted(acc, 2 * e + 298, m * m);
    }
    keys[r] = bad ? NAN : round_to_double(acc);
  }
}
