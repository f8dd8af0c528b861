// Host side of the library: argument validation, the megabatch plan
// (workspace layout, per-phase tile tables, operand scales) and the phase
// sequence of Gram Newton-Schulz, then the C ABI declared in include/dion.h.
//
// The phase sequence follows the Gram form of Newton-Schulz described in the
// Dion3 summary (方法 / 核心模块, "Gram Newton-Schulz" bullet): G = X X^T,
// then per iteration P = aI + bG + cG^2, Q <- P Q, and either G <- P G P or,
// at a restart, X <- Q X, G <- X X^T, Q <- I; finally out = Q X.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <deque>
#include <functional>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/dion.h"
#include "dion_internal.h"
#include "lowrank_internal.h"

namespace dion {
// launchers (gemm_kernels.hip, stream_kernels.hip)
bool launch_gemm16(int bm, int na, int nb, int epi, bool sym, const GemmLaunch& L, const PhaseArgs& pa,
                   hipStream_t stream);
bool launch_gemm64(int epi, bool sym, const GemmLaunch& L, const PhaseArgs& pa, hipStream_t stream);
void launch_rowkeys(int fmt, bool exact, const MatDesc* descs, int nmat, int64_t rows, double* keys,
                    hipStream_t s);
void launch_momentum_keys(bool grad_bf16, bool exact, const MatDesc* descs, int nmat, int64_t rows, float beta,
                          double* keys, int write_out, hipStream_t s);
void launch_update_unselected(bool w_bf16, const MatDesc* descs, int nmat, int64_t rows, const uint8_t* flags,
                              float keep, bool raw, hipStream_t s);
void launch_decay_selected(const MatDesc* descs, int nmat, int64_t total_sel, const int* idx, float beta,
                           hipStream_t s);
void launch_select(const MatDesc* descs, int nmat, const double* keys, uint8_t* flags, int* idx,
                   MatScalars* scalars, bool fp64_path, hipStream_t s);
void launch_pack(int fmt, bool fp64_path, const MatDesc* descs, const int* mats, const int* prefix, int nmat,
                 int total, const int* idx, const MatScalars* scalars, int xterms, bool use_idx, hipStream_t s);
void launch_transpose(const MatDesc* descs, const int* mats, const int* prefix, int nmat, int total, int src_slot,
                      int dst_slot, hipStream_t s);
void launch_copy_unselected(bool bf16, const MatDesc* descs, int nmat, int64_t rows, const uint8_t* flags,
                            hipStream_t s);
void launch_unpack(bool fp64_path, const MatDesc* descs, const int* prefix, int nmat, int total, int slot,
                   const MatScalars* scalars, float scale, bool use_nu2, hipStream_t s);
void launch_scale_combine(MatScalars* scalars, int nmat, hipStream_t s);
void launch_upload(void* dst, const void* src, size_t bytes, hipStream_t s);
void launch_tiny_gns(const MatDesc* descs, const int* ids, int ntiny, const MatScalars* scalars, const int* idx,
                     const double* coef, int K, unsigned long long restarts, int in_fmt, int out_fmt, int update,
                     float keep, hipStream_t s);
// matrices with Gram side m <= 64 and long side n <= 1024, or m <= 16 and any
// long side up to 2^24, run in one fp64 launch
constexpr int kTinyM = 64, kTinyN = 1024, kTinyMLong = 16, kTinyNMax = 1 << 24;
inline bool tiny_shape(int m, int n) { return m <= kTinyM && n <= kTinyNMax && (n <= kTinyN || m <= kTinyMLong); }
}  // namespace dion

using namespace dion;

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

const float kQuintic[3] = {3.4445f, -4.7750f, 2.0315f};
constexpr int kMaxIter = 64;
// The MFMA16 path's error grows with the iterations: each one scales the
// rounding in the small singular directions by its slope a_k (safety folded
// in).  Its 2e-2 gate is established up to twelve iterations whose slopes
// multiply to at most the fixed quintic's 3.4445^12 and, for schedules kept as
// given with a run of more than two iterations, runs of at most five
// iterations between restarts and slopes multiplying to at most 3.4445^6 (a
// kept run ahead of further iterations reached 2.5-3.2e-2 at eight iterations
// of the fixed quintic, where the cut schedule stays under 7e-3); calls that
// would put a matrix on that path beyond this are refused (the FP64 path takes
// them).
constexpr int kMfmaMaxIter = 12, kMfmaMaxKeptRun = 5;

// A GEMM phase takes 256-row tiles (one block per CU) when they number at
// least four waves of the 256 CUs, else 128-row tiles (two blocks per CU).
// Between two and four waves the smaller tiles measured faster: the final
// apply of the GPT-2-small batch (972 tiles of 256) 0.21 -> 0.16 ms, its
// other phases unchanged.
constexpr long long kBigTileMinTiles = 1024;
const double kMfmaMaxGain = std::pow(3.4445, 12), kMfmaMaxKeptGain = std::pow(3.4445, 6);

// ------------------------------------------------------------ parameters
struct Params {
  std::vector<double> a, b, c;  // per iteration, safety folded in
  std::vector<int> restart;     // restart[k-1] = 1: restart after iteration k
  double row_frac;
  bool fp64;
  bool carry;   // row-subset step: the carry form of error feedback
  bool keep_schedule;  // MFMA16: run long segments as given (two-term chain)
};

bool valid_dtype(int dtype) { return dtype == DION_BF16 || dtype == DION_FP32 || dtype == DION_FP16; }
size_t dtype_bytes(int dtype) { return dtype == DION_FP32 ? 4 : 2; }

int parse_params(const dion_ns_params* p, int dtype, bool step_mode, Params& out) {
  if (!p) return fail(DION_E_INVAL, "params is NULL");
  if (!valid_dtype(dtype)) return fail(DION_E_INVAL, "unknown dtype");
  if (p->n_iter < 1 || p->n_iter > kMaxIter) return fail(DION_E_INVAL, "n_iter must be in [1, 64]");
  const int K = p->n_iter;
  const float* co = p->ns_coeffs ? p->ns_coeffs : kQuintic;
  const int sets = p->ns_coeffs ? p->n_coeff_sets : 1;
  if (sets != 1 && sets != K) return fail(DION_E_INVAL, "n_coeff_sets must be 1 or n_iter");
  if (!(p->safety > 0.f) || !std::isfinite(p->safety)) return fail(DION_E_INVAL, "safety must be finite and > 0");
  if (!(p->row_frac > 0.f && p->row_frac <= 1.f)) return fail(DION_E_INVAL, "row_frac must be in (0, 1]");
  if (p->restart_every < 0) return fail(DION_E_INVAL, "restart_every must be >= 0");
  if (p->precision < DION_PREC_AUTO || p->precision > DION_PREC_FP64) return fail(DION_E_INVAL, "unknown precision");
  if (step_mode && p->precision == DION_PREC_FP64)
    return fail(DION_E_UNSUPPORTED, "the row-subset step runs on the MFMA16 path only");
  out.a.resize(K);
  out.b.resize(K);
  out.c.resize(K);
  out.restart.assign(K, 0);
  const double s = p->safety;
  for (int k = 0; k < K; ++k) {
    const float* t = co + 3 * (sets == 1 ? 0 : k);
    if (!std::isfinite(t[0]) || !std::isfinite(t[1]) || !std::isfinite(t[2]))
      return fail(DION_E_INVAL, "coefficients must be finite");
    out.a[k] = (double)t[0] / s;
    out.b[k] = (double)t[1] / (s * s * s);
    out.c[k] = (double)t[2] / (s * s * s * s * s);
  }
  if (!std::isfinite(p->restart_threshold) || p->restart_threshold < 0.f)
    return fail(DION_E_INVAL, "restart_threshold must be finite and >= 0");
  const bool by_threshold = !p->restart_mask && p->restart_threshold > 0.f;
  double growth = 1.0;  // product of a_k^2 since the last restart
  for (int k = 1; k < K; ++k) {  // never after the last iteration
    bool r;
    if (p->restart_mask) {
      r = k <= 32 && ((p->restart_mask >> (k - 1)) & 1u);
    } else if (by_threshold) {
      growth *= out.a[k - 1] * out.a[k - 1];
      r = growth >= (double)p->restart_threshold;
      if (r) growth = 1.0;
    } else {
      r = p->restart_every > 0 && k % p->restart_every == 0;
    }
    out.restart[k - 1] = r ? 1 : 0;
  }
  if (p->ef_carry != 0 && p->ef_carry != 1) return fail(DION_E_INVAL, "ef_carry must be 0 or 1");
  out.carry = p->ef_carry == 1;
  if (p->keep_schedule != 0 && p->keep_schedule != 1) return fail(DION_E_INVAL, "keep_schedule must be 0 or 1");
  out.keep_schedule = p->keep_schedule == 1;
  out.row_frac = p->row_frac;
  out.fp64 = p->precision == DION_PREC_FP64 || (p->precision == DION_PREC_AUTO && dtype == DION_FP32 && !step_mode);
  return DION_OK;
}

int selected_count(int R, double frac) {
  const double x = frac * (double)R;
  long long k = (long long)std::ceil(x * (1.0 - 1e-6));
  if (k < 1) k = 1;
  if (k > R) k = R;
  return (int)k;
}

// ----------------------------------------------- scalar bounds (MFMA16)
// Power-of-two scales keep every stored fp16 operand within range: each
// quantity's spectral norm (>= its largest entry) is bounded by pushing the
// singular-value bound of the iterate through the scalar polynomial.
double poly_max(double a, double b, double c, double lam_max, int mode) {
  // mode 0: max |a + b l + c l^2|, mode 1: max |l (a + b l + c l^2)|, over l in [0, lam_max]
  double best = 0.0;
  const int N = 4096;
  for (int i = 0; i <= N; ++i) {
    const double l = lam_max * i / N;
    double v = a + b * l + c * l * l;
    if (mode == 1) v *= l;
    best = std::max(best, std::fabs(v));
  }
  return best * 1.02 + 1e-30;
}
double sv_max(double a, double b, double c, double s_max) {  // max |f(s)| on [0, s_max]
  double best = 0.0;
  const int N = 4096;
  for (int i = 0; i <= N; ++i) {
    const double x = s_max * i / N;
    best = std::max(best, std::fabs(a * x + b * x * x * x + c * x * x * x * x * x));
  }
  return best * 1.02 + 1e-30;
}
float pow2_scale(double bound) {  // largest 2^j with bound * 2^j <= 2^15
  int j = (int)std::floor(std::log2(32768.0 / bound));
  j = std::max(-60, std::min(60, j));
  return std::ldexp(1.0f, j);
}

// ------------------------------------------------------------ the plan
enum StepKind { ST_KEYS, ST_MOMENTUM, ST_SELECT, ST_PACK, ST_GEMM, ST_TRANSPOSE, ST_COPY, ST_UNPACK, ST_COMBINE,
                ST_UPDATE, ST_TINY, ST_DECAY };

struct Step {
  StepKind kind;
  int bm = 0, na = 1, nb = 1, epi = 0;
  bool sym = false;
  int table = 0;  // index into Plan::tabs
  PhaseArgs pa{};
  int src_slot = 0, dst_slot = 0;
  int dset = 0;          // phase entry points: 0 = the matrices, 1 = the apply's Q operands
  int ranges = -1;       // ST_GEMM: index of its 9 tile-range starts in Plan::range_ints
  int grid = 0;          // ST_GEMM: blocks launched
  float scale = 1.f;     // ST_UNPACK: value scale (times nu^2 when use_nu2)
  bool use_nu2 = false;
  // accounting for profiles: name, useful FLOPs (the caller's schedule, by the
  // per-unit formulas), algorithmic FLOPs (the same formulas over every product
  // the plan runs: also the accumulated restart factor and the restarts a cut
  // schedule adds), executed MFMA FLOPs, algorithmic bytes
  const char* name = "";
  double useful = 0, alg = 0, raw = 0, bytes = 0;
};

struct Table {  // a (matrix list, prefix) pair inside the int blob
  size_t mats_off = 0, prefix_off = 0;  // in ints
  int nmat = 0, total = 0;
};

struct MatPlan {
  int R, C, k, m, n, m_pad, n_pad, tall;
  bool acc;  // restarts after the first start from X0 with the accumulated factor
  bool acc_sym = false;  // ... with S = Q_2 Q_1 as a mirrored product
  bool tiny = false;  // runs in the one-workgroup fp64 kernel
  size_t off[N_SLOTS];
  size_t bytes = 0;   // its buffers in the workspace
};

struct Plan {
  bool fp64 = false;
  bool bf16_in = true;   // 16-bit inputs (bf16 or fp16): exact in one fp16 term
  int fmt = 0;           // input storage: 0 bf16, 1 fp32, 2 fp16
  int xterms0 = 1;
  bool use_idx = false;
  // row keys rounded exactly (they decide a selection, or are an output);
  // otherwise they only give ||M||_F^2 and the plain fp64 sum serves
  bool exact_keys = false;
  std::vector<MatPlan> mats;
  int64_t total_rows = 0, total_sel = 0;
  // phase entry points: a second descriptor set (the apply's Q operands, one
  // per matrix, rows counted after the matrices' rows), host-written scalars
  int nq = 0;
  int64_t x_rows = 0, x_sel = 0;
  bool host_scalars = false;
  std::vector<MatScalars> hscal;
  // every matrix small: the whole iteration in one launch (k_tiny_gns), with
  // the per-iteration coefficients (fp64, as int pairs) at ints[coef_off]
  bool tiny = false;      // every matrix takes k_tiny_gns: the plan is that one launch
  int ntiny = 0;          // matrices taking k_tiny_gns; their ids at ints[tiny_ids_off]
  size_t tiny_ids_off = 0;
  size_t coef_off = 0;
  unsigned long long restarts = 0;
  int K = 0;
  // row-subset step with the carry form of error feedback
  bool carry = false;
  // fused weight update (row-subset step): out is the weight W
  bool update = false, w_bf16 = true;
  float keep = 1.f;
  size_t off_descs = 0, off_scalars = 0, off_keys = 0, off_flags = 0, off_idx = 0, off_ints = 0,
         off_data = 0, total = 0, upload_bytes = 0;
  // per GEMM launch, the 9 starts of its 8 per-XCD tile ranges (uploaded
  // with the header; room for max_ranges launches is reserved at layout time)
  size_t off_ranges = 0;
  int max_ranges = 0;
  std::vector<int> range_ints;
  int bm[4] = {0, 0, 0, 0};   // tile sizes of the symmetric, restart-apply, full and final products
  std::vector<int> ints;
  std::vector<Table> tabs;
  std::vector<Step> steps;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Splits a GEMM launch's tiles into 8 contiguous ranges, one per XCD, of
// equal work: a tile costs its reduction depth K plus a fixed 512 for its
// prologue and epilogue.  Batches grouped by shape (all the long-K matrices
// last, say) would otherwise leave most of the work to one XCD.
void balance_ranges(Plan& P, int table, const PhaseArgs& pa, Step& g);

int add_table(Plan& P, const std::vector<int>& mats, const std::vector<int>& counts) {
  Table t;
  t.nmat = (int)mats.size();
  t.mats_off = P.ints.size();
  P.ints.insert(P.ints.end(), mats.begin(), mats.end());
  t.prefix_off = P.ints.size();
  int acc = 0;
  for (int c : counts) {
    P.ints.push_back(acc);
    acc += c;
  }
  P.ints.push_back(acc);
  t.total = acc;
  P.tabs.push_back(t);
  return (int)P.tabs.size() - 1;
}

void balance_ranges(Plan& P, int table, const PhaseArgs& pa, Step& g) {
  const Table& tb = P.tabs[table];
  const int* mats = P.ints.data() + tb.mats_off;
  const int* prefix = P.ints.data() + tb.prefix_off;
  std::vector<double> cost(tb.nmat);
  double total = 0.0;
  for (int j = 0; j < tb.nmat; ++j) {
    const MatPlan& mp = P.mats[mats[j]];
    cost[j] = (double)(pa.k_is_n ? mp.n_pad : mp.m_pad) + 512.0;
    total += cost[j] * (prefix[j + 1] - prefix[j]);
  }
  int r[9];
  r[0] = 0;
  r[8] = tb.total;
  double cum = 0.0;  // work of the matrices before j
  int j = 0;
  for (int x = 1; x < 8; ++x) {
    const double target = total * x / 8.0;
    while (j < tb.nmat && cum + cost[j] * (prefix[j + 1] - prefix[j]) < target) {
      cum += cost[j] * (prefix[j + 1] - prefix[j]);
      ++j;
    }
    int t = tb.total;
    if (j < tb.nmat) t = prefix[j] + (int)std::ceil((target - cum) / cost[j]);
    r[x] = std::min(std::max(t, r[x - 1]), tb.total);
  }
  int widest = 0;
  for (int x = 0; x < 8; ++x) widest = std::max(widest, r[x + 1] - r[x]);
  g.ranges = (int)(P.range_ints.size() / 9);
  g.grid = 8 * widest;
  P.range_ints.insert(P.range_ints.end(), r, r + 9);
}

// bm_force: the four tile sizes to use (a wave of a larger call takes the
// whole call's, so that its results are bit-identical), or NULL to choose
int build_plan(const dion_shape* shapes, int batch, int dtype, const Params& prm, bool step_mode, Plan& P,
               int grad_es = 2, const int* bm_force = nullptr) {
  if (!shapes) return fail(DION_E_INVAL, "shapes is NULL");
  if (batch < 1) return fail(DION_E_INVAL, "batch must be >= 1");
  P.fp64 = prm.fp64;
  P.fmt = step_mode ? 1 : (dtype == DION_FP32 ? 1 : (dtype == DION_FP16 ? 2 : 0));
  P.bf16_in = P.fmt != 1;
  P.xterms0 = (P.fp64 || P.bf16_in) ? 1 : 2;  // bf16 and fp16 values are exact in one fp16 term
  P.use_idx = prm.row_frac < 1.0;
  P.exact_keys = P.use_idx;
  const int K = (int)prm.a.size();
  // The restarts the GEMM schedule runs: the caller's and, on the MFMA16 path
  // unless keep_schedule is set, one more after every second iteration of a
  // longer run between restarts.  A restart re-forms G from the current
  // iterate, so the result is the same in exact arithmetic; only the rounding
  // changes.  Runs of at most two iterations take one-term fp16 operands in
  // their m x m chain, whose rounding does not get to compound; a longer run
  // needs two terms, about three times the MFMA work of its chain and of the
  // final apply, where a restart costs one apply and one Gram.  Useful FLOPs
  // are counted on the caller's schedule: the added restarts' products are
  // extra work.
  std::vector<int> xr = prm.restart;
  if (!P.fp64 && !prm.keep_schedule) {
    int k0 = 0;  // the current run started after iteration k0
    for (int k = 1; k < K; ++k) {
      if (!xr[k - 1] && k - k0 == 2) xr[k - 1] = 2;   // 2 = added here
      if (xr[k - 1]) k0 = k;
    }
  }
  int n_restarts = 0;
  for (int r : xr) n_restarts += (r != 0);
  const bool any_restart = n_restarts > 0;
  // The one-term chain's symmetric-in-exact-arithmetic products (Q <- P Q,
  // and the accumulated restart factor S = Q_2 Q_1) are mirrored when the
  // slopes of the whole schedule multiply to at most six iterations of the
  // fixed quintic's (every configured workload): the mirrored triangle's
  // rounding is then amplified by few iterations afterwards.
  double gain_all = 1.0;
  for (int k = 0; k < K; ++k) gain_all *= std::max(1.0, std::fabs(prm.a[k]));
  const bool mirror_q = !P.fp64 && gain_all <= std::pow(3.4445, 6) * (1.0 + 1e-9);
  // S is mirrored only where every run between restarts is short (at most two
  // iterations, the default cut): a kept longer run gives Q_1 the gain of
  // every one of its iterations, and the mirror's wrong-side rounding with it
  // (a kept five-iteration run, K = 8: 3.3e-2 mirrored, within the gate full)
  bool all_short = true;
  {
    int k0 = 0;
    for (int k = 1; k <= K; ++k)
      if (k == K || xr[k - 1]) {
        if (k - k0 > 2) all_short = false;
        k0 = k;
      }
  }
  const bool mirror_s = mirror_q && all_short;
  const size_t es = P.fp64 ? 8 : 2;
  const size_t mm_terms = P.fp64 ? 1 : 2;
  const size_t xt_terms = P.fp64 ? 1 : 2;

  P.mats.resize(batch);
  for (int i = 0; i < batch; ++i) {
    const int R = shapes[i].rows, C = shapes[i].cols;
    if (R < 1 || C < 1) return fail(DION_E_INVAL, "matrix " + std::to_string(i) + ": rows and cols must be >= 1");
    if ((int64_t)R * C > ((int64_t)1 << 40)) return fail(DION_E_INVAL, "matrix too large");
    MatPlan& mp = P.mats[i];
    mp.R = R;
    mp.C = C;
    mp.k = selected_count(R, prm.row_frac);
    mp.tall = mp.k > C;
    mp.m = std::min(mp.k, C);
    mp.n = std::max(mp.k, C);
    mp.m_pad = pad_up(mp.m);
    mp.n_pad = pad_up(mp.n);
    // At the second restart, X_2 = Q_2 X_1 can be formed as (Q_2 Q_1) X0:
    // X0 is exact in one fp16 term (bf16 input), so the apply takes one term
    // instead of the iterate's two, at the price of one m x m product.  That
    // pays where the apply's long side dominates.  Only in schedules of
    // exactly two restarts: the accumulated factor is rounded to one term at
    // every accumulation and carries the gain of every iteration since X0, so
    // with more restarts its rounding compounds (emulation, K = 7 or 8 with
    // restarts every 2 or every iteration: 1.0-2.4e-2 against 1.8-7.8e-3
    // restarting from the two-term iterate).
    // Cost per matrix: S as a full product (2m^3) plus the one-term apply
    // (2m^2 n) against the two-term apply (4m^2 n), i.e. n >= 1.5m; a
    // mirrored S costs m^3, which pays for every shape (n >= m).  Gram sides
    // below 128 rows keep the full product: they average out the mirror's
    // wrong-side rounding least, and its saving there is negligible.
    mp.acc_sym = mirror_s && mp.m >= 128;
    mp.acc = !P.fp64 && P.xterms0 == 1 && n_restarts == 2 &&
             (mp.acc_sym || 2 * (int64_t)mp.n >= 3 * (int64_t)mp.m);
    mp.acc_sym = mp.acc_sym && mp.acc;
    P.total_rows += R;
    P.total_sel += mp.k;
  }
  P.x_rows = P.total_rows;
  P.x_sel = P.total_sel;
  size_t off = 0;
  P.off_descs = off;
  off = align256(off + sizeof(MatDesc) * batch);

  // Matrices small enough for the one-workgroup fp64 kernel (k_tiny_gns)
  // take it: all of them, and the plan is that one launch, or some, and they
  // take it beside the GEMM phases of the others (the "mf" list below).  On
  // the MFMA path they would occupy 256-row tiles for a few rows, and a Gram
  // side of a few rows cannot average out the fp16 rounding of its small
  // singular direction (errors near 2e-2 for two rows).
  std::vector<int> mf, tiny_ids;
  for (int i = 0; i < batch; ++i) {
    MatPlan& mp = P.mats[i];
    mp.tiny = tiny_shape(mp.m, mp.n);
    (mp.tiny ? tiny_ids : mf).push_back(i);
  }
  P.tiny = mf.empty();
  if (!P.fp64 && !mf.empty()) {
    double gain = 1.0;
    for (int k = 0; k < K; ++k) gain *= std::max(1.0, std::fabs(prm.a[k]));
    int run = 0, longest = 0;
    for (int k = 1; k <= K; ++k) {
      ++run;
      if (k == K || prm.restart[k - 1]) {
        longest = std::max(longest, run);
        run = 0;
      }
    }
    if (K > kMfmaMaxIter || gain > kMfmaMaxGain * (1.0 + 1e-9))
      return fail(DION_E_UNSUPPORTED, "the MFMA16 path holds its error bound up to 12 iterations with slopes a_k "
                                      "multiplying to at most 3.4445^12; use DION_PREC_FP64");
    if (prm.keep_schedule && longest > 2 &&
        (longest > kMfmaMaxKeptRun || gain > kMfmaMaxKeptGain * (1.0 + 1e-9)))
      return fail(DION_E_UNSUPPORTED, "keep_schedule: a run of more than 5 iterations between restarts, or a kept "
                                      "run in a schedule whose slopes a_k multiply to more than 3.4445^6, is "
                                      "outside the MFMA16 path's error bound; use keep_schedule = 0 or DION_PREC_FP64");
  }

  // tables of the GEMM phases, over mf
  auto sym_counts = [&](int bm) {
    std::vector<int> c;
    for (int i : mf) { int T = P.mats[i].m_pad / bm; c.push_back(T * (T + 1) / 2); }
    return c;
  };
  auto rect_counts = [&](const std::vector<int>& ms, int bm, bool rows_n) {
    std::vector<int> c;
    for (int i : ms) {
      const MatPlan& mp = P.mats[i];
      c.push_back((rows_n ? mp.n_pad : mp.m_pad) / bm * ((rows_n ? mp.m_pad : mp.n_pad) / bm));
    }
    return c;
  };
  auto total_of = [](const std::vector<int>& c) { long long s = 0; for (int x : c) s += x; return s; };
  // tile size per phase kind: 256 when it gives at least kBigTileMinTiles blocks
  auto pick_bm = [&](std::function<std::vector<int>(int)> counts) {
    if (P.fp64) return 64;
    return total_of(counts(256)) >= kBigTileMinTiles ? 256 : 128;
  };
  const int bm_sym = bm_force ? bm_force[0] : pick_bm([&](int bm) { return sym_counts(bm); });
  const int bm_xtq = bm_force ? bm_force[1] : pick_bm([&](int bm) { return rect_counts(mf, bm, true); });
  auto full_counts = [&](int bm) {
    std::vector<int> c;
    for (int i : mf) { int T = P.mats[i].m_pad / bm; c.push_back(T * T); }
    return c;
  };
  const int bm_full = bm_force ? bm_force[2] : pick_bm([&](int bm) { return full_counts(bm); });
  std::vector<int> wide, tall, accs, naccs;
  for (int i : mf) (P.mats[i].tall ? tall : wide).push_back(i);
  for (int i : mf) (P.mats[i].acc ? accs : naccs).push_back(i);
  const bool any_acc = !accs.empty();
  const int bm_fin = bm_force ? bm_force[3] : pick_bm([&](int bm) {
    auto a = rect_counts(wide, bm, false), b = rect_counts(tall, bm, true);
    a.insert(a.end(), b.begin(), b.end());
    return a;
  });
  P.bm[0] = bm_sym;
  P.bm[1] = bm_xtq;
  P.bm[2] = bm_full;
  P.bm[3] = bm_fin;
  const int t_sym = add_table(P, mf, sym_counts(bm_sym));
  const int t_xtq = add_table(P, mf, rect_counts(mf, bm_xtq, true));
  const int t_full = add_table(P, mf, full_counts(bm_full));
  const int t_wide = add_table(P, wide, rect_counts(wide, bm_fin, false));
  const int t_tall = add_table(P, tall, rect_counts(tall, bm_fin, true));
  // restarts after the first: matrices that restart from X0 and the others
  auto sub_full = [&](const std::vector<int>& ms, int bm) {
    std::vector<int> c;
    for (int i : ms) { int T = P.mats[i].m_pad / bm; c.push_back(T * T); }
    return c;
  };
  const int t_xtq_acc = add_table(P, accs, rect_counts(accs, bm_xtq, true));
  const int t_xtq_nacc = add_table(P, naccs, rect_counts(naccs, bm_xtq, true));
  const int t_full_acc = add_table(P, accs, sub_full(accs, bm_full));
  auto sub_sym = [&](const std::vector<int>& ms, int bm) {
    std::vector<int> c;
    for (int i : ms) { int T = P.mats[i].m_pad / bm; c.push_back(T * (T + 1) / 2); }
    return c;
  };
  std::vector<int> accs_sym, accs_full;   // S mirrored, or run in full
  for (int i : accs) (P.mats[i].acc_sym ? accs_sym : accs_full).push_back(i);
  const int t_sym_acc = add_table(P, accs_sym, sub_sym(accs_sym, bm_sym));
  const int t_full_acc_s = add_table(P, accs_full, sub_full(accs_full, bm_full));
  const int t_full_nacc = add_table(P, naccs, sub_full(naccs, bm_full));
  // pack and transpose tables over the MFMA matrices (the kernels look the
  // matrices up through the table's list)
  std::vector<int> pack_c;
  for (int i : mf) pack_c.push_back((P.mats[i].m_pad / 64) * (P.mats[i].n_pad / 64));  // k_pad C_pad = m_pad n_pad
  const int t_pack = add_table(P, mf, pack_c);
  const int t_tr = add_table(P, mf, pack_c);
  P.K = K;
  if (!tiny_ids.empty()) {
    P.ntiny = (int)tiny_ids.size();
    P.tiny_ids_off = P.ints.size();
    P.ints.insert(P.ints.end(), tiny_ids.begin(), tiny_ids.end());
    if (P.ints.size() & 1) P.ints.push_back(0);   // 8-byte alignment of the fp64 table
    P.coef_off = P.ints.size();
    for (int k = 0; k < K; ++k)
      for (double v : {prm.a[k], prm.b[k], prm.c[k]}) {
        int w[2];
        std::memcpy(w, &v, sizeof v);
        P.ints.push_back(w[0]);
        P.ints.push_back(w[1]);
      }
    for (int k = 1; k < K; ++k)
      if (prm.restart[k - 1]) P.restarts |= 1ull << (k - 1);
  }
  // uploaded part: descriptors, tables, tile ranges; then device-written scratch
  P.off_ints = off;
  off = align256(off + sizeof(int) * P.ints.size());
  P.max_ranges = 16 + 8 * K;   // more than the GEMM launches of any plan below
  P.off_ranges = off;
  off = align256(off + sizeof(int) * 9 * P.max_ranges);
  P.upload_bytes = off;
  P.off_scalars = off; off = align256(off + sizeof(MatScalars) * batch);
  P.off_keys = off;    off = align256(off + sizeof(double) * P.total_rows);
  P.off_flags = off;   off = align256(off + P.total_rows);
  P.off_idx = off;     off = align256(off + sizeof(int) * P.total_sel);

  // per-matrix buffers
  P.off_data = off;
  for (int i = 0; i < batch; ++i) {
    MatPlan& mp = P.mats[i];
    const size_t mn = (size_t)mp.m_pad * mp.n_pad, mm = (size_t)mp.m_pad * mp.m_pad;
    const size_t first = off;
    for (int s = 0; s < N_SLOTS; ++s) mp.off[s] = 0;
    if (mp.tiny) {   // k_tiny_gns: the iterate and its restart copy, m x n fp64 each
      const size_t x = (size_t)mp.m * mp.n * 8;
      mp.off[SLOT_X] = off;   off = align256(off + x);
      mp.off[SLOT_XT0] = off; off = align256(off + x);
      mp.bytes = off - first;
      continue;
    }
    mp.off[SLOT_X] = off;   off = align256(off + mn * es);
    mp.off[SLOT_XT0] = off; off = align256(off + mn * es * xt_terms);
    if (any_restart) {
      mp.off[SLOT_XT1] = off; off = align256(off + mn * es * xt_terms);
      mp.off[SLOT_XTE] = mp.acc ? mp.off[SLOT_XT1] : mp.off[SLOT_XT0];
    }
    const int last_mm = any_acc ? SLOT_MM5 : SLOT_MM3;
    for (int s = SLOT_MM0; s <= last_mm; ++s) { mp.off[s] = off; off = align256(off + mm * es * mm_terms); }
    mp.bytes = off - first;
  }
  P.total = off;

  // ---------------------------------------------------------- phase list
  const double in_es = step_mode ? 4.0 : (double)dtype_bytes(dtype);
  double elems = 0, sel_elems = 0, pad_elems = 0, unsel_elems = 0, rows = (double)P.total_rows;
  for (const MatPlan& mp : P.mats) {
    elems += (double)mp.R * mp.C;
    sel_elems += (double)mp.k * mp.C;
    if (!mp.tiny) pad_elems += (double)mp.m_pad * mp.n_pad;
    unsel_elems += (double)(mp.R - mp.k) * mp.C;
  }
  Step st;
  st.kind = step_mode ? ST_MOMENTUM : ST_KEYS;
  st.name = step_mode ? "momentum" : "rowkeys";
  st.bytes = step_mode ? elems * (4 + 4 + grad_es + 2) + rows * 8 : elems * in_es + rows * 8;
  P.steps.push_back(st);
  st = Step();
  st.kind = ST_SELECT;
  st.name = "select";
  st.bytes = rows * 8 * (P.use_idx ? 10 : 1) + rows;
  P.steps.push_back(st);
  if (P.ntiny) {
    // useful FLOPs per segment of length L: n m (m + 1) + 2 m^2 n + (4L - 3) m^2 (m + 1)
    st = Step();
    st.kind = ST_TINY;
    st.name = "tiny";
    for (int i : tiny_ids) {
      const MatPlan& mp = P.mats[i];
      const double m = mp.m, n = mp.n;
      int k0 = 0;
      for (int k = 1; k <= K; ++k)
        if (k == K || prm.restart[k - 1]) {
          const double L = k - k0;
          st.useful += n * m * (m + 1) + 2.0 * m * m * n + (4.0 * L - 3.0) * m * m * (m + 1);
          k0 = k;
        }
      st.bytes += 2.0 * mp.k * mp.C * in_es;
    }
    st.raw = st.alg = st.useful;
    P.steps.push_back(st);
  }
  P.carry = step_mode && prm.carry;
  auto decay = [&]() {   // carry: the captured rows of the buffer decay once read
    Step dc;
    dc.kind = ST_DECAY;
    dc.name = "decay_rows";
    dc.bytes = 8.0 * sel_elems;
    P.steps.push_back(dc);
  };
  if (P.tiny) {
    if (P.carry) decay();
    if (P.use_idx && !step_mode) {
      Step cp;
      cp.kind = ST_COPY;
      cp.name = "copy_rows";
      cp.bytes = 2.0 * unsel_elems * in_es + rows;
      P.steps.push_back(cp);
    }
    return DION_OK;
  }
  st = Step();
  st.kind = ST_PACK;
  st.name = "pack";
  st.table = t_pack;
  st.bytes = sel_elems * in_es + pad_elems * es * (1 + P.xterms0);
  P.steps.push_back(st);
  if (P.carry) decay();

  // per-matrix useful FLOPs of a product kind; executed MFMA FLOPs from the tile table
  // out_lo: whether any later product or epilogue reads the lo term of this
  // product's fp16 output (skipping it halves the output stores)
  auto gemm = [&](int table, int bm, bool sym, int na, int nb, int epi, PhaseArgs pa, const char* name,
                  bool out_lo, bool counts_useful = true) {
    pa.out_lo = out_lo ? 1 : 0;
    Step g;
    g.name = name;
    const Table& tb = P.tabs[table];
    const int nprod = P.fp64 ? 1 : ((na == 2 && nb == 2) ? 3 : ((na == 2 || nb == 2) ? 2 : 1));
    for (int j = 0; j < tb.nmat; ++j) {
      const MatPlan& mp = P.mats[P.ints[tb.mats_off + j]];
      const double m = mp.m, n = mp.n;
      const int tiles = P.ints[tb.prefix_off + j + 1] - P.ints[tb.prefix_off + j];
      const double K = pa.k_is_n ? mp.n_pad : mp.m_pad;
      g.raw += (double)tiles * bm * bm * K * 2.0 * nprod;
      // an m x m chain product counts as the symmetric half however it is run
      const bool mxm = !pa.k_is_n && !pa.a_rows_is_n && !pa.b_rows_is_n && epi != EPI_OUT;
      const double f = (sym && pa.k_is_n) ? n * m * (m + 1)      // Gram
                       : mxm ? m * m * (m + 1)                    // m x m chain
                       : 2.0 * m * m * n;                         // apply / final
      g.alg += f;
      if (counts_useful) g.useful += f;                           // else extra work of the execution
      // algorithmic HBM bytes on the padded layout: every operand term read
      // once, the result written once (both triangles of a symmetric one)
      const double ar = pa.a_rows_is_n ? mp.n_pad : mp.m_pad, br = pa.b_rows_is_n ? mp.n_pad : mp.m_pad;
      const double el = P.fp64 ? 8.0 : 2.0, to = P.fp64 ? 1.0 : 2.0;
      g.bytes += el * K * (ar * (P.fp64 ? 1 : na) + br * (P.fp64 ? 1 : nb));
      const double mm = (double)mp.m_pad * mp.m_pad;
      const double tw = (P.fp64 || out_lo) ? to : 1.0;             // output terms written
      if (epi == EPI_SYM) g.bytes += el * tw * mm;
      else if (epi == EPI_POLY) g.bytes += el * (to + tw) * mm;     // reads G (both terms), writes P
      else if (epi == EPI_RECT) g.bytes += el * tw * ar * br;
      else if (epi == EPI_RECT_T) g.bytes += el * (tw + 1.0) * ar * br;
      else g.bytes += (pa.out_fp32 ? 4.0 : 2.0) * m * n;
    }
    g.kind = ST_GEMM;
    g.table = table;
    balance_ranges(P, table, pa, g);
    g.bm = bm;
    g.sym = sym;
    g.na = P.fp64 ? 1 : na;
    g.nb = P.fp64 ? 1 : nb;
    g.epi = epi;
    g.pa = pa;
    P.steps.push_back(g);
  };
  auto sc = [&](double bound) { return P.fp64 ? 1.0f : pow2_scale(bound); };

  double sb = 1.0;  // bound on the singular values of the current iterate
  int g_slot = SLOT_MM0;
  float sG = sc(sb * sb);
  // operand terms of the m x m chain in the segment that starts after
  // iteration k0 (a restart, or k0 = 0): one for segments of at most two
  // iterations, two for longer ones (see the policy below)
  auto seg_terms = [&](int k0) {
    int e = k0 + 1;
    while (e < K && !xr[e - 1]) ++e;
    return (P.fp64 || e - k0 > 2) ? 2 : 1;
  };
  {
    PhaseArgs pa{};
    pa.a_slot = pa.b_slot = SLOT_X;
    pa.c_slot = g_slot;
    pa.k_is_n = 1;
    pa.alpha = sG;
    pa.alpha_pow = 2;
    // G's lo term is read only by a segment that runs two-term
    gemm(t_sym, bm_sym, true, 1, 1, EPI_SYM, pa, "syrk", seg_terms(0) == 2);
  }
  // the m x m slots not holding G; an exhausted list fails the plan below
  // rather than handing out a slot twice
  std::vector<int> freel = {SLOT_MM3, SLOT_MM2, SLOT_MM1};
  if (any_acc) freel.insert(freel.begin(), {SLOT_MM5, SLOT_MM4});
  bool out_of_slots = false;
  auto take = [&]() {
    if (freel.empty()) {
      out_of_slots = true;
      return (int)SLOT_MM1;
    }
    const int v = freel.back();
    freel.pop_back();
    return v;
  };
  int q_slot = -1, xt_slot = SLOT_XT0, xterms = P.xterms0;
  float sQ = 1.f, sXT = 1.f;
  double qb = 1.0;
  int n_rest = 0;         // restarts taken so far
  int qa_slot = -1;       // accumulated factor: Q_1, then S = Q_2 Q_1 (matrices restarting from X0)
  int qat_slot = -1;      // Q_1^T (hi term), or qa_slot when Q_1 is exactly symmetric
  int pending_qat = -1;   // Q_1^T written by the product that forms Q_1
  float sQA = 1.f;
  double qab = 1.0;
  bool x_is_x0 = true;
  int ct = 2;         // operand terms of the m x m chain products in this segment
  bool short_seg = false;  // one-term chain: Q <- P Q as a full (unmirrored) product
  // ... or mirrored, when the schedule's slopes multiply to at most six
  // iterations of the fixed quintic's (every configured workload): the
  // mirrored triangle's rounding is amplified by fewer iterations afterwards
  for (int k = 1; k <= K; ++k) {
    const double a = prm.a[k - 1], b = prm.b[k - 1], c = prm.c[k - 1];
    if (q_slot < 0) {
      // A segment runs from a (re)start to the next restart or the last
      // iteration.  The fp16 rounding of a one-term operand enters G through
      // every P G P update and is amplified by the polynomial's slope at the
      // small singular values, so it compounds with the segment's length: a
      // segment of one or two iterations (at most one G update) takes
      // one-term chain products, longer segments two terms.  The restart
      // apply keeps X in two terms in every case.
      //
      // With one-term operands the product Q <- P Q is symmetric in exact
      // arithmetic (P and Q are polynomials in the same Gram matrix), but its
      // rounding error is not: in the eigenbasis the error of entry (i, j)
      // carries the weights of row i, and a mirror copies the entries whose
      // row is a small singular direction (where P is near its slope
      // a = 3.4445) into the transposed position, which the apply Q X then
      // multiplies by the large singular values, and every later iteration
      // by its slope.  So it is mirrored (half the work) only when the slopes
      // of the whole schedule multiply to at most six iterations of the fixed
      // quintic's, and run in full otherwise.  T = P G is always mirrored: its
      // error is only half as harmful, since the next product P T^T is
      // Gram-shaped.  Emulation against the oracle (Llama-shaped 1024 x 4096,
      // restarts every 2): relative error 5.6e-3 with both products full,
      // 6.3e-3 with T mirrored, 9.1e-3 with both mirrored; on the row-subset
      // blocks 3.7e-3, 5.9e-3 and 1.2e-2.  Measured on the GPU with both
      // mirrored: 7.1-7.2e-3 on the Llama-3-8B samples (5.5-5.9e-3 with Q
      // full), 5.2-6.2e-3 on the row-subset blocks (gate 2e-2), for 4.5% less
      // time on that batch.
      int e = k;
      while (e < K && !xr[e - 1]) ++e;
      ct = e - k + 1 <= 2 ? 1 : 2;
      short_seg = !P.fp64 && ct == 1;
    }
    const double gb = sb * sb;
    const double pb = poly_max(a, b, c, gb, 0), tb = poly_max(a, b, c, gb, 1);
    const double sb_next = sv_max(a, b, c, sb);
    const float sP = sc(pb);
    const int p_slot = take();
    {  // P = a I + b G + c G^2, fused into the G*G epilogue
      PhaseArgs pa{};
      pa.a_slot = pa.b_slot = pa.aux_slot = g_slot;
      pa.c_slot = p_slot;
      pa.alpha = 1.0f / (sG * sG);
      pa.poly_a = (float)a;
      pa.poly_b = (float)b;
      pa.poly_c = (float)c;
      pa.aux_inv_scale = 1.0f / sG;
      pa.aux_lo = ct == 2 ? 1 : 0;
      pa.out_scale = sP;
      // G*G takes the segment's operand terms, and so does the bG term of
      // the epilogue.  In a one-term segment bG then reads the same rounding
      // of G as the product, so P is a polynomial of one matrix: emulated
      // error 6.0e-3 against 6.3e-3 with a two-term bG (Llama-shaped
      // 1024 x 4096), and G's lo term is never stored.  In a long segment a
      // one-term G*G even at the segment's first iteration doubles the error
      // of the segments that follow a restart (emulation: 1.5e-2 -> 7.4e-3 on
      // 256 x 256 with a restart after iteration 2 of 5).
      gemm(t_sym, bm_sym, true, ct, ct, EPI_POLY, pa, "gram_poly", ct == 2);
    }
    if (q_slot < 0) {
      q_slot = p_slot;
      sQ = sP;
      qb = pb;
    } else {  // Q <- P Q
      const double qb_new = qb * pb;
      const float sQn = sc(qb_new);
      const int qn = take();
      PhaseArgs pa{};
      pa.a_slot = p_slot;
      pa.b_slot = q_slot;
      pa.c_slot = qn;
      pa.alpha = sQn / (sP * sQ);
      if (short_seg && mirror_q) {   // symmetric in exact arithmetic: the upper triangle and its mirror
        gemm(t_sym, bm_sym, true, 1, 1, EPI_SYM, pa, "sym_product", false);
      } else if (short_seg && any_acc && k < K && xr[k - 1] && n_rest == 0) {
        // this Q starts the accumulated factor of the matrices restarting
        // from X0; the accumulation at the second restart multiplies by it
        // from the right, which reads its rows as columns: keep Q^T (hi) as well
        pending_qat = take();
        PhaseArgs pt = pa;
        pt.aux_slot = pending_qat;
        gemm(t_full_acc, bm_full, false, 1, 1, EPI_RECT_T, pt, "full_product", false);
        if (P.tabs[t_full_nacc].nmat) gemm(t_full_nacc, bm_full, false, 1, 1, EPI_RECT, pa, "full_product", false);
      } else if (short_seg) {
        gemm(t_full, bm_full, false, 1, 1, EPI_RECT, pa, "full_product", false);
      } else {
        gemm(t_sym, bm_sym, true, ct, ct, EPI_SYM, pa, "sym_product", true);
      }
      freel.push_back(q_slot);
      q_slot = qn;
      sQ = sQn;
      qb = qb_new;
    }
    if (k == K) break;
    if (xr[k - 1]) {
      // X <- Q X, computed as X'^T = X^T Q; then X = transpose; G = X X^T.
      // P is dead here (the apply and the accumulation read Q and X): its slot
      // goes back first, so that the accumulation's two new slots fit beside
      // G, Q, S and S^T in the six m x m slots
      if (p_slot != q_slot) freel.push_back(p_slot);
      ++n_rest;
      const bool added = xr[k - 1] == 2;   // a restart of the schedule policy: extra work
      const float sXn = sc(sb_next);
      // odd-numbered restarts write XT1, even-numbered ones XTE (XT0's buffer,
      // or XT1's for matrices restarting from X0, whose X0^T stays in XT0)
      const int xt_new = (n_rest & 1) ? SLOT_XT1 : SLOT_XTE;
      // X^T is read in two terms by the next restart apply, or by the final
      // apply, which takes its hi term only after a short last segment.
      // Matrices restarting from X0 read it only in the final apply.
      int e2 = k + 1;
      while (e2 < K && !xr[e2 - 1]) ++e2;
      const bool xt_lo = !(e2 == K && e2 - k <= 2);
      const bool xt_lo_acc = xt_lo && e2 == K;
      auto apply = [&](int table, int a_slot, int na, int b_slot, float alpha, int alpha_pow, bool lo) {
        PhaseArgs pa{};
        pa.a_slot = a_slot;
        pa.b_slot = b_slot;
        pa.c_slot = xt_new;
        pa.a_rows_is_n = 1;
        pa.alpha = alpha;
        pa.alpha_pow = alpha_pow;
        // MFMA16: the epilogue also writes X (hi) transposed; FP64: a transpose pass
        pa.aux_slot = SLOT_X;
        gemm(table, bm_xtq, false, na, 1, P.fp64 ? EPI_RECT : EPI_RECT_T, pa, "apply", lo, !added);
      };
      const float al = x_is_x0 ? sXn / sQ : sXn / (sXT * sQ);
      const int alp = x_is_x0 ? 1 : 0;
      if (!any_acc) {
        apply(t_xtq, xt_slot, xterms, q_slot, al, alp, xt_lo);
      } else if (n_rest == 1) {  // the same product, split by who reads the lo term
        apply(t_xtq_acc, xt_slot, xterms, q_slot, al, alp, xt_lo_acc);
        if (P.tabs[t_xtq_nacc].nmat) apply(t_xtq_nacc, xt_slot, xterms, q_slot, al, alp, xt_lo);
      } else {
        // the second (and last) restart of the matrices restarting from X0:
        // S = Q_2 Q_1 (a full one-term product in this order, outside the
        // useful count; it reads Q_1^T by rows), then X'^T = X0^T S^T
        const double qab_new = qab * qb;
        const float sQAn = sc(qab_new);
        const int qa_new = take();
        PhaseArgs pq{};
        pq.a_slot = q_slot;
        pq.b_slot = qat_slot;
        pq.c_slot = qa_new;
        pq.alpha = sQAn / (sQ * sQA);
        // where Q_1 and Q_2 are mirrored, S is symmetric in exact arithmetic
        if (P.tabs[t_sym_acc].nmat) gemm(t_sym_acc, bm_sym, true, 1, 1, EPI_SYM, pq, "acc_product", false, false);
        if (P.tabs[t_full_acc_s].nmat) gemm(t_full_acc_s, bm_full, false, 1, 1, EPI_RECT, pq, "acc_product", false, false);
        freel.push_back(qa_slot);
        if (qat_slot != qa_slot) freel.push_back(qat_slot);
        qa_slot = qat_slot = qa_new;
        sQA = sQAn;
        qab = qab_new;
        apply(t_xtq_acc, SLOT_XT0, 1, qa_slot, sXn / sQA, 1, xt_lo_acc);
        if (P.tabs[t_xtq_nacc].nmat) apply(t_xtq_nacc, xt_slot, xterms, q_slot, al, alp, xt_lo);
      }
      if (P.fp64) {
        Step tr;
        tr.kind = ST_TRANSPOSE;
        tr.table = t_tr;
        tr.src_slot = xt_new;
        tr.dst_slot = SLOT_X;
        tr.name = "transpose";
        tr.bytes = 2.0 * pad_elems * es;
        P.steps.push_back(tr);
      }
      const float sGn = sc(sb_next * sb_next);
      {
        PhaseArgs pa{};
        pa.a_slot = pa.b_slot = SLOT_X;
        pa.c_slot = g_slot;
        pa.k_is_n = 1;
        pa.alpha = sGn / (sXn * sXn);
        gemm(t_sym, bm_sym, true, 1, 1, EPI_SYM, pa, "syrk", seg_terms(k) == 2, !added);
      }
      sG = sGn;
      xt_slot = xt_new;
      xterms = P.fp64 ? 1 : 2;
      sXT = sXn;
      x_is_x0 = false;
      if (n_rest == 1 && any_acc) {  // Q_1 starts the accumulated factor
        qa_slot = q_slot;
        qat_slot = pending_qat >= 0 ? pending_qat : q_slot;  // else Q_1 is exactly symmetric
        sQA = sQ;
        qab = qb;
      } else {
        freel.push_back(q_slot);
      }
      q_slot = -1;
    } else {
      // G <- P T^T with T = P G, i.e. P G P (each product reads B by rows: C = A B^T)
      const float sT = sc(tb);
      const int t_slot = take();
      {
        PhaseArgs pa{};
        pa.a_slot = p_slot;
        pa.b_slot = g_slot;
        pa.c_slot = t_slot;
        pa.alpha = sT / (sP * sG);
        // the lo term of T is read only by a two-term P T^T
        gemm(t_sym, bm_sym, true, ct, ct, EPI_SYM, pa, "sym_product", ct == 2);
      }
      const float sGn = sc(sb_next * sb_next);
      {
        PhaseArgs pa{};
        pa.a_slot = p_slot;
        pa.b_slot = t_slot;
        pa.c_slot = g_slot;
        pa.alpha = sGn / (sP * sT);
        gemm(t_sym, bm_sym, true, ct, ct, EPI_SYM, pa, "sym_product", ct == 2);
      }
      sG = sGn;
      freel.push_back(t_slot);
      if (p_slot != q_slot) freel.push_back(p_slot);
    }
    sb = sb_next;
  }
  if (out_of_slots) return fail(DION_E_UNSUPPORTED, "internal: the schedule needs more m x m buffers");
  {  // out = Q X: wide matrices as Q * X, tall ones as X^T * Q
    // After a short last segment both operands enter in their hi term: Q's
    // gain there is at most about a^2 and nothing amplifies the rounding
    // afterwards (emulation: +1e-4 of relative error).  After a long one Q
    // carries the gain of every iteration of the segment and its one-term
    // rounding dominates the output error, so Q takes both terms, and X too
    // when it has two (emulation: 1.0e-2 -> 1.7e-3 without restarts, 7.4e-3 ->
    // 2.7e-3 with a restart after iteration 2 of 5).
    const int fx = short_seg ? 1 : xterms;
    const int fq = (short_seg || P.fp64) ? 1 : 2;
    PhaseArgs pa{};
    pa.alpha = x_is_x0 ? 1.0f / sQ : 1.0f / (sQ * sXT);
    pa.alpha_pow = x_is_x0 ? 1 : 0;
    pa.out_fp32 = (!step_mode && dtype == DION_FP32) ? 1 : 0;
    pa.out_f16 = (!step_mode && dtype == DION_FP16) ? 1 : 0;
    PhaseArgs pw = pa;
    pw.a_slot = q_slot;
    pw.b_slot = xt_slot;
    pw.b_rows_is_n = 1;
    pw.out_rows_are_m = 1;
    if (P.tabs[t_wide].nmat) gemm(t_wide, bm_fin, false, fq, fx, EPI_OUT, pw, "final", false);
    PhaseArgs pt = pa;
    pt.a_slot = xt_slot;
    pt.b_slot = q_slot;
    pt.a_rows_is_n = 1;
    pt.out_rows_are_m = 0;
    if (P.tabs[t_tall].nmat) gemm(t_tall, bm_fin, false, fx, fq, EPI_OUT, pt, "final", false);
  }
  if (P.use_idx && !step_mode) {
    Step cp;
    cp.kind = ST_COPY;
    cp.name = "copy_rows";
    cp.bytes = 2.0 * unsel_elems * in_es + rows;
    P.steps.push_back(cp);
  }
  if ((int)P.range_ints.size() > 9 * P.max_ranges)
    return fail(DION_E_UNSUPPORTED, "internal: more GEMM launches than reserved tile ranges");
  return DION_OK;
}

// ------------------------------------------------- phase entry points
// One phase of the path on its own, for kernel-level checks: the same
// kernels, descriptors and workspace layout as the full plan, with an unpack
// of the m x m result to fp32 where the phase's output is internal.
enum PhaseKind { PH_KEYS = 1, PH_SYRK = 2, PH_POLY = 3, PH_APPLY = 4 };

bool phase_fp64(int precision, int dtype) {
  return precision == DION_PREC_FP64 || (precision == DION_PREC_AUTO && dtype == DION_FP32);
}

int build_phase_plan(int ph, const dion_shape* shapes, int batch, int dtype, int precision, double row_frac,
                     const float* coeffs, Plan& P) {
  if (!shapes) return fail(DION_E_INVAL, "shapes is NULL");
  if (batch < 1) return fail(DION_E_INVAL, "batch must be >= 1");
  if (!valid_dtype(dtype)) return fail(DION_E_INVAL, "unknown dtype");
  if (precision < DION_PREC_AUTO || precision > DION_PREC_FP64) return fail(DION_E_INVAL, "unknown precision");
  if (!(row_frac > 0.0 && row_frac <= 1.0)) return fail(DION_E_INVAL, "row_frac must be in (0, 1]");
  P.fp64 = phase_fp64(precision, dtype);
  P.fmt = dtype == DION_FP32 ? 1 : (dtype == DION_FP16 ? 2 : 0);
  P.bf16_in = P.fmt != 1;
  P.xterms0 = (P.fp64 || P.bf16_in) ? 1 : 2;
  P.use_idx = row_frac < 1.0;
  P.exact_keys = ph == PH_KEYS || P.use_idx;
  P.mats.resize(batch);
  for (int i = 0; i < batch; ++i) {
    const int R = shapes[i].rows, C = shapes[i].cols;
    if (R < 1 || C < 1) return fail(DION_E_INVAL, "matrix " + std::to_string(i) + ": rows and cols must be >= 1");
    if ((int64_t)R * C > ((int64_t)1 << 40)) return fail(DION_E_INVAL, "matrix too large");
    if (ph == PH_POLY && R != C) return fail(DION_E_INVAL, "matrix " + std::to_string(i) + " must be square");
    MatPlan& mp = P.mats[i];
    mp.R = R;
    mp.C = C;
    mp.k = selected_count(R, row_frac);
    mp.tall = mp.k > C;
    mp.m = std::min(mp.k, C);
    mp.n = std::max(mp.k, C);
    mp.m_pad = pad_up(mp.m);
    mp.n_pad = pad_up(mp.n);
    mp.acc = false;
    for (int s2 = 0; s2 < N_SLOTS; ++s2) mp.off[s2] = 0;
    P.total_rows += R;
    P.total_sel += mp.k;
  }
  P.x_rows = P.total_rows;
  P.x_sel = P.total_sel;
  if (ph == PH_APPLY) {
    P.nq = batch;
    for (const MatPlan& mp : P.mats) {
      P.total_rows += mp.m;
      P.total_sel += mp.m;
    }
  }
  const int ndesc = batch + P.nq;
  const size_t es = P.fp64 ? 8 : 2;
  const size_t terms = P.fp64 ? 1 : 2;

  std::vector<int> all(batch), wide, tall;
  for (int i = 0; i < batch; ++i) {
    all[i] = i;
    (P.mats[i].tall ? tall : wide).push_back(i);
  }
  auto counts = [&](const std::vector<int>& ms, std::function<int(const MatPlan&)> f) {
    std::vector<int> c;
    for (int i : ms) c.push_back(f(P.mats[i]));
    return c;
  };
  auto total_of = [](const std::vector<int>& c) { long long t = 0; for (int x : c) t += x; return t; };
  auto pick = [&](std::function<std::vector<int>(int)> cnt) {
    if (P.fp64) return 64;
    return total_of(cnt(256)) >= kBigTileMinTiles ? 256 : 128;
  };
  const int t_pack = add_table(P, all, counts(all, [](const MatPlan& mp) { return (mp.m_pad / 64) * (mp.n_pad / 64); }));
  const int t_mm64 = add_table(P, all, counts(all, [](const MatPlan& mp) { return (mp.m_pad / 64) * (mp.m_pad / 64); }));
  const int bm_sym = pick([&](int bm) {
    return counts(all, [bm](const MatPlan& mp) { const int T = mp.m_pad / bm; return T * (T + 1) / 2; });
  });
  const int t_sym = add_table(P, all, counts(all, [bm_sym](const MatPlan& mp) {
    const int T = mp.m_pad / bm_sym; return T * (T + 1) / 2; }));
  auto rect = [&](const std::vector<int>& ms, int bm) {
    return counts(ms, [bm](const MatPlan& mp) { return (mp.m_pad / bm) * (mp.n_pad / bm); });
  };
  const int bm_fin = pick([&](int bm) {
    auto a = rect(wide, bm), b = rect(tall, bm);
    a.insert(a.end(), b.begin(), b.end());
    return a;
  });
  const int t_wide = add_table(P, wide, rect(wide, bm_fin));
  const int t_tall = add_table(P, tall, rect(tall, bm_fin));

  size_t off = 0;
  P.off_descs = off;
  off = align256(off + sizeof(MatDesc) * ndesc);
  P.off_ints = off;
  off = align256(off + sizeof(int) * P.ints.size());
  P.max_ranges = 16;
  P.off_ranges = off;
  off = align256(off + sizeof(int) * 9 * P.max_ranges);
  if (ph == PH_POLY) {  // the operand scale is known on the host: ||G||_2 <= 1
    P.host_scalars = true;
    P.off_scalars = off;
    off = align256(off + sizeof(MatScalars) * ndesc);
    P.hscal.resize(ndesc);
    for (MatScalars& sc : P.hscal) {
      sc.nu2 = 1.0;
      sc.e = P.fp64 ? 0 : 14;  // |G_ij| <= 1 -> |G_ij * 2^14| <= 2^14
      sc.x0_alpha64 = std::ldexp(1.0, -sc.e);
      sc.x0_alpha = (float)sc.x0_alpha64;
    }
  }
  P.upload_bytes = off;
  if (ph != PH_POLY) {
    P.off_scalars = off;
    off = align256(off + sizeof(MatScalars) * ndesc);
  }
  P.off_keys = off;  off = align256(off + sizeof(double) * P.total_rows);
  P.off_flags = off; off = align256(off + P.total_rows);
  P.off_idx = off;   off = align256(off + sizeof(int) * P.total_sel);
  P.off_data = off;
  if (ph != PH_KEYS) {
    for (MatPlan& mp : P.mats) {
      const size_t mn = (size_t)mp.m_pad * mp.n_pad, mm = (size_t)mp.m_pad * mp.m_pad;
      mp.off[SLOT_X] = off;   off = align256(off + mn * es);
      mp.off[SLOT_XT0] = off; off = align256(off + mn * es * terms);
      mp.off[SLOT_MM0] = off; off = align256(off + mm * es * terms);
      if (ph == PH_APPLY) { mp.off[SLOT_MM1] = off; off = align256(off + mm * es * terms); }
    }
  }
  P.total = off;

  auto step = [&](StepKind kind, const char* name, int dset = 0, int table = 0) {
    Step st;
    st.kind = kind;
    st.name = name;
    st.dset = dset;
    st.table = table;
    P.steps.push_back(st);
    return &P.steps.back();
  };
  auto gemm = [&](int table, int bm, bool sym, int na, int nb, int epi, const PhaseArgs& pa, const char* name) {
    Step* g = step(ST_GEMM, name, 0, table);
    g->bm = bm;
    g->sym = sym;
    g->na = P.fp64 ? 1 : na;
    g->nb = P.fp64 ? 1 : nb;
    g->epi = epi;
    g->pa = pa;
    g->pa.out_lo = 1;
    balance_ranges(P, table, pa, *g);
  };
  const float sG = P.fp64 ? 1.f : pow2_scale(1.0);
  if (ph == PH_KEYS || ph == PH_SYRK || ph == PH_APPLY) {
    step(ST_KEYS, "rowkeys");
    step(ST_SELECT, "select");
  }
  if (ph == PH_APPLY) {
    step(ST_KEYS, "rowkeys", 1);
    step(ST_SELECT, "select", 1);
    step(ST_COMBINE, "combine");
    step(ST_PACK, "pack", 1, t_mm64);
  }
  if (ph != PH_KEYS) step(ST_PACK, "pack", 0, t_pack);
  if (ph == PH_SYRK) {  // G = X X^T / nu^2 (one fp16 term of X), unpacked times nu^2
    PhaseArgs pa{};
    pa.a_slot = pa.b_slot = SLOT_X;
    pa.c_slot = SLOT_MM0;
    pa.k_is_n = 1;
    pa.alpha = sG;
    pa.alpha_pow = 2;
    gemm(t_sym, bm_sym, true, 1, 1, EPI_SYM, pa, "syrk");
    Step* u = step(ST_UNPACK, "unpack", 0, t_mm64);
    u->src_slot = SLOT_MM0;
    u->scale = 1.f / sG;
    u->use_nu2 = true;
  } else if (ph == PH_POLY) {  // P = a I + b G + c G^2 from G^T in XT0 (two terms)
    const double a = coeffs[0], b = coeffs[1], c = coeffs[2];
    const float sP = P.fp64 ? 1.f : pow2_scale(std::fabs(a) + std::fabs(b) + std::fabs(c));
    const float sX = (float)P.hscal[0].x0_alpha64;
    PhaseArgs pa{};
    pa.a_slot = pa.b_slot = pa.aux_slot = SLOT_XT0;
    pa.c_slot = SLOT_MM0;
    pa.alpha = sX * sX;
    pa.poly_a = (float)a;
    pa.poly_b = (float)b;
    pa.poly_c = (float)c;
    pa.aux_inv_scale = sX;
    pa.aux_lo = 1;
    pa.out_scale = sP;
    gemm(t_sym, bm_sym, true, 2, 2, EPI_POLY, pa, "gram_poly");
    Step* u = step(ST_UNPACK, "unpack", 0, t_mm64);
    u->src_slot = SLOT_MM0;
    u->scale = 1.f / sP;
  } else if (ph == PH_APPLY) {  // Y = Q X (wide) or X Q (tall), scale 2^-(e_X + e_Q)
    PhaseArgs pa{};
    pa.alpha = 1.f;
    pa.alpha_pow = 1;
    pa.out_fp32 = dtype == DION_FP32 ? 1 : 0;
    pa.out_f16 = dtype == DION_FP16 ? 1 : 0;
    PhaseArgs pw = pa;
    pw.a_slot = SLOT_MM0;
    pw.b_slot = SLOT_XT0;
    pw.b_rows_is_n = 1;
    pw.out_rows_are_m = 1;
    if (!wide.empty()) gemm(t_wide, bm_fin, false, 2, P.xterms0, EPI_OUT, pw, "final");
    PhaseArgs pt = pa;
    pt.a_slot = SLOT_XT0;
    pt.b_slot = SLOT_MM0;
    pt.a_rows_is_n = 1;
    pt.out_rows_are_m = 0;
    if (!tall.empty()) gemm(t_tall, bm_fin, false, P.xterms0, 2, EPI_OUT, pt, "final");
  }
  if ((int)P.range_ints.size() > 9 * P.max_ranges)
    return fail(DION_E_UNSUPPORTED, "internal: more GEMM launches than reserved tile ranges");
  return DION_OK;
}

// ---------------------------------------------------- pinned upload stage
// The plan header goes to the device from a pinned host buffer with one
// asynchronous copy.  A buffer may be refilled once the stream has passed its
// copy (its event has completed); the host never waits for that.  The ring
// grows to kStageSlots buffers when the host runs ahead of the device, and
// beyond that the header travels as kernel arguments (launch_upload), which
// needs no buffer at all.
constexpr int kStageSlots = 8;
struct Stage {
  void* host[kStageSlots] = {};
  size_t cap[kStageSlots] = {};
  hipEvent_t ev[kStageSlots] = {};
  int n = 0;      // slots in use
  int next = 0;   // where the search for a free slot starts
};
thread_local Stage g_stage;

int hip_fail(const char* what, hipError_t e) {
  return fail(DION_E_HIP, std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")");
}

int upload(const void* src, size_t bytes, void* dst, hipStream_t s) {
  Stage& S = g_stage;
  hipError_t e;
  int slot = -1;
  for (int j = 0; j < S.n && slot < 0; ++j) {   // a slot whose last copy has completed
    const int i = (S.next + j) % S.n;
    e = hipEventQuery(S.ev[i]);
    if (e == hipSuccess) slot = i;
    else if (e != hipErrorNotReady) return hip_fail("hipEventQuery", e);
  }
  if (slot < 0 && S.n < kStageSlots) {          // none free: one more slot
    slot = S.n;
    if ((e = hipEventCreateWithFlags(&S.ev[slot], hipEventDisableTiming)) != hipSuccess) {
      S.ev[slot] = nullptr;
      return hip_fail("hipEventCreateWithFlags", e);
    }
    ++S.n;
  }
  if (slot < 0) {                               // the host is kStageSlots calls ahead
    launch_upload(dst, src, bytes, s);
    return DION_OK;
  }
  S.next = (slot + 1) % S.n;
  if (S.cap[slot] < bytes) {
    if (S.host[slot]) (void)hipHostFree(S.host[slot]);
    S.host[slot] = nullptr;
    S.cap[slot] = 0;
    const size_t cap = std::max(bytes, (size_t)1 << 16);
    if ((e = hipHostMalloc(&S.host[slot], cap, hipHostMallocDefault)) != hipSuccess)
      return hip_fail("hipHostMalloc of the upload stage", e);
    S.cap[slot] = cap;
  }
  std::memcpy(S.host[slot], src, bytes);
  if ((e = hipMemcpyAsync(dst, S.host[slot], bytes, hipMemcpyHostToDevice, s)) != hipSuccess)
    return hip_fail("hipMemcpyAsync of the plan", e);
  if ((e = hipEventRecord(S.ev[slot], s)) != hipSuccess) return hip_fail("hipEventRecord", e);
  return DION_OK;
}

// ------------------------------------------------------------ profiling
// While enabled, each phase launch of the calling thread is bracketed by two
// hipEvents recorded on the call's stream; records keep the phase's
// accounting so callers can turn durations into rates.
struct ProfRec {
  const char* name;
  const char* kernel;
  hipEvent_t a, b;
  double useful, raw, bytes, alg;
};

// Name of the kernel instance a step launches, as the profiler prints it
// (template arguments included); s_fmt is the element format the step reads
// (0 bf16, 1 fp32, 2 fp16), grad_bf16 the row-subset step's gradient type.
const char* kernel_name(const Plan& P, const Step& st, int s_fmt, bool grad_bf16) {
  thread_local std::deque<std::string> cache;  // stable addresses
  const char* in_t = s_fmt == 1 ? "float" : (s_fmt == 2 ? "_Float16" : "unsigned short");
  std::string key;
  switch (st.kind) {
    case ST_KEYS: key = std::string("dion::k_rowkeys<") + in_t + (P.exact_keys ? ", true>" : ", false>"); break;
    case ST_MOMENTUM:
      key = std::string(grad_bf16 ? "dion::k_momentum_keys<unsigned short" : "dion::k_momentum_keys<float") +
            (P.exact_keys ? ", true>" : ", false>");
      break;
    case ST_SELECT: key = "dion::k_select"; break;
    case ST_PACK: key = std::string(P.fp64 ? "dion::k_pack<" : "dion::k_pack16<") + in_t + ">"; break;
    case ST_TRANSPOSE: key = "dion::k_transpose<double>"; break;
    case ST_COPY: key = s_fmt != 1 ? "dion::k_copy_unselected<unsigned short>" : "dion::k_copy_unselected<float>"; break;
    case ST_TINY: key = "dion::k_tiny_gns"; break;
    case ST_DECAY: key = "dion::k_decay_selected"; break;
    case ST_UNPACK: key = P.fp64 ? "dion::k_unpack<double>" : "dion::k_unpack<_Float16>"; break;
    case ST_COMBINE: key = "dion::k_scale_combine"; break;
    case ST_UPDATE:
      key = P.w_bf16 ? "dion::k_update_unselected<unsigned short>" : "dion::k_update_unselected<float>";
      break;
    case ST_GEMM:
      if (P.fp64)
        key = "dion::k_gemm64<" + std::to_string(st.epi) + ", " + (st.sym ? "true" : "false") + ">";
      else
        key = "dion::k_gemm16<" + std::to_string(st.bm) + ", " + std::to_string(st.na) + ", " +
              std::to_string(st.nb) + ", " + std::to_string(st.epi) + ", " + (st.sym ? "true" : "false") + ">";
      break;
  }
  for (const std::string& k : cache)
    if (k == key) return k.c_str();
  cache.push_back(key);
  return cache.back().c_str();
}
struct Profiler {
  bool on = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  void clear() {
    for (auto& r : recs) {
      pool.push_back(r.a);
      pool.push_back(r.b);
    }
    recs.clear();
  }
};
thread_local Profiler g_prof;

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char* pa = (const char*)a;
  const char* pb = (const char*)b;
  return pa < pb + nb && pb < pa + na;
}

// by_value: upload the plan header as kernel arguments (no pinned staging
// buffer), for the allocation-free entry point
int run(const Plan& P, const void* const* M, void* const* out, const void* const* grad, int batch, int dtype,
        int grad_dtype, float beta, bool step_mode, int32_t* sel_idx, void* workspace, size_t ws_bytes,
        hipStream_t stream, const void* const* Qs = nullptr, double* keys_out = nullptr,
        const float* upd_alpha = nullptr, bool by_value = false) {
  if (!workspace) return fail(DION_E_WORKSPACE, "workspace is NULL");
  if (((uintptr_t)workspace & 255) != 0) return fail(DION_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < P.total)
    return fail(DION_E_WORKSPACE, "workspace too small: need " + std::to_string(P.total) + " bytes");
  char* ws = (char*)workspace;
  // descriptors
  std::vector<char> blob(P.upload_bytes, 0);
  MatDesc* descs = (MatDesc*)blob.data();
  int64_t row0 = 0, sel0 = 0;
  for (int i = 0; i < batch; ++i) {
    const MatPlan& mp = P.mats[i];
    MatDesc& d = descs[i];
    d.M = M[i];
    d.out = out ? out[i] : nullptr;
    d.grad = grad ? grad[i] : nullptr;
    for (int s = 0; s < N_SLOTS; ++s) d.buf[s] = mp.off[s] ? ws + mp.off[s] : nullptr;
    d.row0 = row0;
    d.sel0 = sel0;
    d.R = mp.R;
    d.C = mp.C;
    d.k = mp.k;
    d.m = mp.m;
    d.n = mp.n;
    d.m_pad = mp.m_pad;
    d.n_pad = mp.n_pad;
    d.tall = mp.tall;
    d.upd_alpha = upd_alpha ? upd_alpha[i] : 0.f;
    row0 += mp.R;
    sel0 += mp.k;
  }
  // the apply's Q operands (m x m fp32): packed as they are into MM0 (two
  // terms) for wide matrices, transposed for tall ones, through the pack's
  // tall / wide roles; their rows, keys and indices are counted from 0
  row0 = sel0 = 0;
  for (int i = 0; i < P.nq; ++i) {
    const MatPlan& mp = P.mats[i];
    MatDesc& d = descs[batch + i];
    d.M = Qs[i];
    d.buf[SLOT_XT0] = ws + mp.off[SLOT_MM0];
    d.buf[SLOT_X] = ws + mp.off[SLOT_MM1];
    d.row0 = row0;
    d.sel0 = sel0;
    d.R = d.C = d.k = d.m = d.n = mp.m;
    d.m_pad = d.n_pad = mp.m_pad;
    d.tall = mp.tall ? 0 : 1;
    row0 += mp.m;
    sel0 += mp.m;
  }
  std::memcpy(blob.data() + P.off_ints, P.ints.data(), sizeof(int) * P.ints.size());
  std::memcpy(blob.data() + P.off_ranges, P.range_ints.data(), sizeof(int) * P.range_ints.size());
  if (P.host_scalars) std::memcpy(blob.data() + P.off_scalars, P.hscal.data(), sizeof(MatScalars) * P.hscal.size());
  if (by_value) {
    launch_upload(ws, blob.data(), blob.size(), stream);
  } else {
    const int rc = upload(blob.data(), blob.size(), ws, stream);
    if (rc) return rc;
  }

  const MatDesc* d_descs = (const MatDesc*)(ws + P.off_descs);
  MatScalars* d_scal = (MatScalars*)(ws + P.off_scalars);
  double* d_keys = (double*)(ws + P.off_keys);
  uint8_t* d_flags = (uint8_t*)(ws + P.off_flags);
  int* d_idx = (int*)(ws + P.off_idx);
  const int* d_ints = (const int*)(ws + P.off_ints);
  const int fmt = P.fmt;

  for (const Step& st : P.steps) {
    ProfRec rec{st.name, nullptr, nullptr, nullptr, st.useful, st.raw, st.bytes, st.alg};
    if (g_prof.on) {
      rec.a = g_prof.get();
      rec.b = g_prof.get();
      if (!rec.a || !rec.b || hipEventRecord(rec.a, stream) != hipSuccess)
        return fail(DION_E_HIP, "profiling event failed");
    }
    // descriptor set of the step: the matrices, or the apply's Q operands
    const bool qset = st.dset == 1;
    const MatDesc* sd = qset ? d_descs + batch : d_descs;
    MatScalars* ss = qset ? d_scal + batch : d_scal;
    const int sn = qset ? P.nq : batch;
    const int64_t srows = qset ? P.total_rows - P.x_rows : P.x_rows;
    double* skeys = qset ? d_keys + P.x_rows : d_keys;
    uint8_t* sflags = qset ? d_flags + P.x_rows : d_flags;
    int* sidx = qset ? d_idx + P.x_sel : d_idx;
    const int s_fmt = qset ? 1 : fmt;   // the apply's Q operands are fp32
    if (g_prof.on) rec.kernel = kernel_name(P, st, s_fmt, grad_dtype == DION_BF16);
    switch (st.kind) {
      case ST_KEYS:
        launch_rowkeys(s_fmt, P.exact_keys && !qset, sd, sn, srows, skeys, stream);
        break;
      case ST_MOMENTUM:
        launch_momentum_keys(grad_dtype == DION_BF16, P.exact_keys, d_descs, batch, P.total_rows, P.carry ? 1.0f : beta,
                             d_keys,
                             P.update ? 0 : (P.carry ? 2 : 1), stream);
        break;
      case ST_SELECT:
        launch_select(sd, sn, skeys, sflags, sidx, ss, P.fp64, stream);
        break;
      case ST_PACK: {
        const Table& t = P.tabs[st.table];
        launch_pack(s_fmt, P.fp64, sd, d_ints + t.mats_off, d_ints + t.prefix_off, t.nmat, t.total, sidx, ss,
                    qset ? 2 : P.xterms0, P.use_idx && !qset, stream);
        break;
      }
      case ST_TRANSPOSE: {
        const Table& t = P.tabs[st.table];
        launch_transpose(d_descs, d_ints + t.mats_off, d_ints + t.prefix_off, t.nmat, t.total, st.src_slot,
                         st.dst_slot, stream);
        break;
      }
      case ST_GEMM: {
        const Table& t = P.tabs[st.table];
        GemmLaunch L{d_descs, d_ints + t.mats_off, d_ints + t.prefix_off, t.nmat, t.total,
                     (const int*)(ws + P.off_ranges) + 9 * st.ranges, st.grid};
        PhaseArgs pa = st.pa;
        pa.scalars = d_scal;
        pa.idx = P.use_idx ? d_idx : nullptr;
        const bool ok = P.fp64 ? launch_gemm64(st.epi, st.sym, L, pa, stream)
                               : launch_gemm16(st.bm, st.na, st.nb, st.epi, st.sym, L, pa, stream);
        if (!ok) return fail(DION_E_UNSUPPORTED, "no GEMM kernel for this phase");
        break;
      }
      case ST_DECAY:
        launch_decay_selected(d_descs, batch, P.total_sel, P.use_idx ? d_idx : nullptr, beta, stream);
        break;
      case ST_TINY:
        // the row-subset step reads the fp32 buffer and writes a bf16 update, or
        // updates the weight in its own dtype
        launch_tiny_gns(d_descs, d_ints + P.tiny_ids_off, P.ntiny, d_scal, P.use_idx ? d_idx : nullptr,
                        (const double*)(d_ints + P.coef_off), P.K, P.restarts, fmt,
                        step_mode ? (P.update && !P.w_bf16 ? 1 : 0) : fmt, P.update ? 1 : 0, P.keep, stream);
        break;
      case ST_COPY:
        launch_copy_unselected(fmt != 1, d_descs, batch, P.total_rows, d_flags, stream);
        break;
      case ST_UNPACK: {
        const Table& t = P.tabs[st.table];
        launch_unpack(P.fp64, d_descs, d_ints + t.prefix_off, t.nmat, t.total, st.src_slot, d_scal, st.scale,
                      st.use_nu2, stream);
        break;
      }
      case ST_COMBINE:
        launch_scale_combine(d_scal, batch, stream);
        break;
      case ST_UPDATE:
        launch_update_unselected(P.w_bf16, d_descs, batch, P.total_rows, d_flags, P.keep, !P.carry, stream);
        break;
    }
    if (g_prof.on) {
      if (hipEventRecord(rec.b, stream) != hipSuccess) return fail(DION_E_HIP, "profiling event failed");
      g_prof.recs.push_back(rec);
    }
  }
  if (sel_idx) {
    if (hipMemcpyAsync(sel_idx, d_idx, sizeof(int) * P.x_sel, hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return fail(DION_E_HIP, "copy of selected indices failed");
  }
  if (keys_out) {
    if (hipMemcpyAsync(keys_out, d_keys, sizeof(double) * P.x_rows, hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return fail(DION_E_HIP, "copy of row keys failed");
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DION_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return DION_OK;
}

int check_ptrs(const void* const* M, void* const* out, const dion_shape* shapes, int batch, size_t esz_in,
               size_t esz_out) {
  if (!M || !out) return fail(DION_E_INVAL, "matrix pointer arrays are NULL");
  for (int i = 0; i < batch; ++i)
    if (!M[i] || !out[i]) return fail(DION_E_INVAL, "matrix " + std::to_string(i) + " has a NULL pointer");
  // out must not overlap any input
  for (int i = 0; i < batch; ++i) {
    const size_t no = (size_t)shapes[i].rows * shapes[i].cols * esz_out;
    for (int j = 0; j < batch; ++j) {
      const size_t ni = (size_t)shapes[j].rows * shapes[j].cols * esz_in;
      if (overlaps(out[i], no, M[j], ni)) return fail(DION_E_INVAL, "out must not overlap the inputs");
    }
  }
  return DION_OK;
}


// ------------------------------------------------------------------ waves
// A call whose workspace is smaller than its whole plan runs as waves:
// consecutive matrices whose own plan fits the workspace, one after another on
// the call's stream (each wave is a full plan: its own selection, Gram
// Newton-Schulz and write-out, all independent per matrix).  Waves take the
// whole call's tile sizes, so the results are bit-identical to one wave.  The
// whole plan bounds each wave's: a wave's header is at most the whole header,
// and each matrix's buffers at most what the whole plan gives it.
struct Wave {
  int i0 = 0, n = 0;   // matrices [i0, i0 + n)
  int64_t sel0 = 0;    // first selected-row entry of the wave
  Plan plan;
};

int plan_waves(const dion_shape* shapes, int batch, int dtype, const Params& prm, bool step_mode, int grad_es,
               size_t budget, std::vector<Wave>& waves, size_t& need) {
  waves.clear();
  waves.emplace_back();
  Plan& full = waves.back().plan;
  int rc = build_plan(shapes, batch, dtype, prm, step_mode, full, grad_es);
  if (rc) return rc;
  waves.back().n = batch;
  need = full.total;
  if (full.total <= budget) return DION_OK;
  const size_t header = full.off_data;
  std::vector<size_t> bytes(batch);
  std::vector<int> ks(batch);
  for (int i = 0; i < batch; ++i) {
    bytes[i] = full.mats[i].bytes;
    ks[i] = full.mats[i].k;
  }
  int bm[4];
  std::memcpy(bm, full.bm, sizeof bm);
  waves.clear();
  need = 0;
  int64_t sel = 0;
  for (int i = 0; i < batch;) {
    size_t acc = header;
    int j = i;
    while (j < batch && acc + bytes[j] <= budget) acc += bytes[j++];
    if (j == i)
      return fail(DION_E_WORKSPACE, "workspace too small: matrix " + std::to_string(i) + " alone needs " +
                                        std::to_string(header + bytes[i]) + " bytes");
    waves.emplace_back();
    Wave& w = waves.back();
    w.i0 = i;
    w.n = j - i;
    w.sel0 = sel;
    rc = build_plan(shapes + i, j - i, dtype, prm, step_mode, w.plan, grad_es, bm);
    if (rc) return rc;
    if (w.plan.total > budget) return fail(DION_E_WORKSPACE, "internal: a wave exceeds its bound");
    need = std::max(need, w.plan.total);
    for (int t = i; t < j; ++t) sel += ks[t];
    i = j;
  }
  return DION_OK;
}

// The row-subset step's fused weight update on a plan: the final apply's
// epilogue updates the selected rows of W, a pass of its own the others.
void make_update(Plan& P, int w_dtype, float weight_decay) {
  P.update = true;
  P.w_bf16 = w_dtype == DION_BF16;
  P.keep = 1.0f - weight_decay;
  const double wes = w_dtype == DION_BF16 ? 2.0 : 4.0;
  // algorithmic bytes: the momentum pass writes no update rows here, and the
  // final apply reads and writes the selected rows of W instead of writing out
  double elems = 0.0, unsel = 0.0;
  for (const MatPlan& mp : P.mats) {
    elems += (double)mp.R * mp.C;
    unsel += (double)(mp.R - mp.k) * mp.C;
  }
  for (Step& st : P.steps) {
    if (st.kind == ST_MOMENTUM) st.bytes -= 2.0 * elems;
    if (st.kind == ST_GEMM && st.epi == EPI_OUT) {
      st.pa.out_update = 1;
      st.pa.upd_keep = P.keep;
      st.pa.out_fp32 = w_dtype == DION_FP32 ? 1 : 0;
      const Table& tb = P.tabs[st.table];
      for (int j = 0; j < tb.nmat; ++j) {
        const MatPlan& mp = P.mats[P.ints[tb.mats_off + j]];
        st.bytes += (2.0 * wes - 2.0) * (double)mp.m * mp.n;
      }
    }
  }
  if (P.use_idx) {
    Step u;
    u.kind = ST_UPDATE;
    u.name = "update_rows";
    u.bytes = unsel * (4.0 + 2.0 * wes) + (double)P.total_rows;   // E read, W read and written; row flags
    P.steps.push_back(u);
  }
}

// ------------------------------------------- low-rank (Dion / Orth-Dion) step
// Orth-Dion explainer, technical summary: one power-iteration step from the
// previous right factor, the residual (error-feedback) buffer, and the right
// factor normalized by columns (Dion) or by QR (Orth-Dion).  Per matrix,
// with r = min(rank, R, C):
//   B = fl32(M + G)                        formed where read (16-bit G), or
//                                          k_lr_accumulate (M in place)
//   P = orth(B Q)                          GEMM, then shifted CholeskyQR3
//   W = B^T P                              GEMM
//   M = B - beta P W^T                     GEMM (beta = -beta, accumulate)
//   Q = orth(W) or colnorm(W)              shifted CholeskyQR3, or k_lr_colnorm
//   out = P Q^T                            GEMM, written in the output dtype
// orth is CholeskyQR run three times, the first on a shifted Gram matrix:
// S = F^T F (GEMM), L = chol(S (+ shift)) and L^-1 in fp64 (k_lr_cholinv),
// F <- F L^-T (GEMM); the triangular factor has a positive diagonal, the QR
// convention of the oracle.  The rank-r products run in k_lr_gemm
// (lowrank_gemm.hip), batched over the matrices of one shape, on two-term
// fp16 operands whose scales come from the max slots (LrSlot) that each
// operand's producer raises; the slots live in the uploaded header, so every
// call starts them at zero (and Dion's normalized Q at one).
constexpr int kMaxRank = 512;
// pointer arrays per group: the matrices' buffers, the max slots, the split
// (fp16 hi and lo) copies of P, W and the new Q, and the gradients
enum { LP_M, LP_Q, LP_X, LP_Y, LP_W, LP_W2, LP_S, LP_L, LP_D, LP_AM, LP_XS, LP_WS, LP_QS, LP_G, LP_N };

struct LrGroup {
  int R, C, r;
  std::vector<int> mats;
  size_t ptr_off;   // LP_N arrays of mats.size() device pointers
};

struct LrPlan {
  std::vector<int> R, C, r;
  std::vector<LrGroup> groups;
  std::vector<int64_t> blk0;
  int64_t blocks = 0;
  bool out_fp32 = false;
  size_t off_descs = 0, off_ptrs = 0, off_amax = 0, off_blockmax = 0, upload_bytes = 0, total = 0;
  std::vector<size_t> off[LP_N];   // per matrix: X, Y, W, W2, S, L
  std::vector<size_t> off_a64;
};

int build_lr_plan(const dion_shape* shapes, int batch, int rank, int out_dtype, LrPlan& P) {
  if (!shapes || batch < 1) return fail(DION_E_INVAL, "shapes must be non-NULL and batch >= 1");
  if (rank < 1) return fail(DION_E_INVAL, "rank must be >= 1");
  if (rank > kMaxRank) return fail(DION_E_UNSUPPORTED, "rank above 512 is not supported");
  if (!valid_dtype(out_dtype)) return fail(DION_E_INVAL, "unknown output dtype");
  P.out_fp32 = out_dtype == DION_FP32;
  std::map<std::tuple<int, int, int>, int> gi;
  P.R.resize(batch); P.C.resize(batch); P.r.resize(batch); P.blk0.resize(batch);
  for (int i = 0; i < batch; ++i) {
    const int R = shapes[i].rows, C = shapes[i].cols;
    if (R < 1 || C < 1) return fail(DION_E_INVAL, "rows and cols must be >= 1");
    const int r = std::min(rank, std::min(R, C));
    P.R[i] = R; P.C[i] = C; P.r[i] = r;
    auto key = std::make_tuple(R, C, r);
    auto it = gi.find(key);
    if (it == gi.end()) {
      gi[key] = (int)P.groups.size();
      P.groups.push_back(LrGroup{R, C, r, {i}, 0});
    } else {
      P.groups[it->second].mats.push_back(i);
    }
    P.blk0[i] = P.blocks;
    P.blocks += ((int64_t)R * C + LR_BLOCK_ELEMS - 1) / LR_BLOCK_ELEMS;
  }
  size_t off = 0;
  P.off_descs = off; off = align256(off + sizeof(LrDesc) * batch);
  P.off_ptrs = off;
  for (LrGroup& g : P.groups) { g.ptr_off = off; off += sizeof(float*) * LP_N * g.mats.size(); }
  off = align256(off);
  P.off_amax = off; off = align256(off + sizeof(unsigned) * LS_N * batch);
  P.upload_bytes = off;
  P.off_blockmax = off; off = align256(off + sizeof(float) * P.blocks);
  for (int k = 0; k < LP_N; ++k) P.off[k].assign(batch, 0);
  P.off_a64.assign(batch, 0);
  for (int i = 0; i < batch; ++i) {
    const size_t R = P.R[i], C = P.C[i], r = P.r[i];
    P.off[LP_X][i] = off;  off = align256(off + 4 * R * r);
    P.off[LP_Y][i] = off;  off = align256(off + 4 * R * r);
    P.off[LP_W][i] = off;  off = align256(off + 4 * C * r);
    P.off[LP_W2][i] = off; off = align256(off + 4 * C * r);
    const size_t parts = (size_t)std::max((R + LR_GRAM_CHUNK - 1) / LR_GRAM_CHUNK, (C + LR_GRAM_CHUNK - 1) / LR_GRAM_CHUNK);
    P.off[LP_S][i] = off;  off = align256(off + 4 * r * r * parts);
    P.off[LP_L][i] = off;  off = align256(off + 4 * r * r);
    P.off_a64[i] = off;    off = align256(off + 8 * r * r);
    const size_t ldp = (r + 31) / 32 * 32, Rp = (R + 127) / 128 * 128, Cp = (C + 127) / 128 * 128;
    P.off[LP_XS][i] = off; off = align256(off + 4 * Rp * ldp);
    P.off[LP_WS][i] = off; off = align256(off + 4 * Cp * ldp);
    P.off[LP_QS][i] = off; off = align256(off + 4 * Cp * ldp);
  }
  P.total = off;
  return DION_OK;
}

int run_lr(const LrPlan& P, float* const* M, const void* const* G, float* const* Q, void* const* out,
           int batch, int grad_dtype, int out_dtype, float beta, int mode, void* workspace, size_t ws_bytes,
           hipStream_t stream) {
  if (!workspace) return fail(DION_E_WORKSPACE, "workspace is NULL");
  if (((uintptr_t)workspace & 255) != 0) return fail(DION_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < P.total) return fail(DION_E_WORKSPACE, "workspace too small: need " + std::to_string(P.total) + " bytes");
  char* ws = (char*)workspace;
  std::vector<char> blob(P.upload_bytes, 0);
  LrDesc* descs = (LrDesc*)(blob.data() + P.off_descs);
  for (int i = 0; i < batch; ++i) {
    LrDesc& d = descs[i];
    d.M = M[i];
    d.G = G[i];
    d.Q = Q[i];
    d.out = out[i];
    d.X = (float*)(ws + P.off[LP_X][i]);
    d.Y = (float*)(ws + P.off[LP_Y][i]);
    d.W = (float*)(ws + P.off[LP_W][i]);
    d.W2 = (float*)(ws + P.off[LP_W2][i]);
    d.S = (float*)(ws + P.off[LP_S][i]);
    d.Linv = (float*)(ws + P.off[LP_L][i]);
    d.A64 = (double*)(ws + P.off_a64[i]);
    d.amax = (unsigned*)(ws + P.off_amax) + (size_t)LS_N * i;
    d.elems = (int64_t)P.R[i] * P.C[i];
    d.blk0 = P.blk0[i];
    d.R = P.R[i];
    d.C = P.C[i];
    d.r = P.r[i];
    d.parts_R = (P.R[i] + LR_GRAM_CHUNK - 1) / LR_GRAM_CHUNK;
    d.parts_C = (P.C[i] + LR_GRAM_CHUNK - 1) / LR_GRAM_CHUNK;
  }
  for (const LrGroup& g : P.groups) {
    float** arr = (float**)(blob.data() + g.ptr_off);
    const size_t n = g.mats.size();
    for (size_t t = 0; t < n; ++t) {
      const LrDesc& d = descs[g.mats[t]];
      const int i = g.mats[t];
      float* const v[LP_N] = {d.M, d.Q, d.X, d.Y, d.W, d.W2, d.S, d.Linv, (float*)d.out, (float*)d.amax,
                              (float*)(ws + P.off[LP_XS][i]), (float*)(ws + P.off[LP_WS][i]),
                              (float*)(ws + P.off[LP_QS][i]), (float*)d.G};
      for (int k = 0; k < LP_N; ++k) arr[k * n + t] = v[k];
    }
  }
  if (mode == DION_LOWRANK_COLNORM) {   // Dion's normalized columns: every |entry| at most one
    unsigned* am = (unsigned*)(blob.data() + P.off_amax);
    for (int i = 0; i < batch; ++i) am[(size_t)LS_N * i + LS_G2] = 0x3F800000u;
  }
  int rc = upload(blob.data(), P.upload_bytes, ws, stream);
  if (rc != DION_OK) return rc;
  const LrDesc* d_descs = (const LrDesc*)(ws + P.off_descs);
  auto arrays = [&](const LrGroup& g, int k) { return (float* const*)(ws + g.ptr_off) + k * g.mats.size(); };
  const int nmat = batch;

  // each launch as one profiling record, with its useful FLOPs (2 m n k per
  // product; also its algorithmic FLOPs) and algorithmic bytes
  auto phase = [&](const char* name, const char* kernel, double useful, double bytes,
                   const std::function<int()>& fn) -> int {
    ProfRec rec{name, kernel, nullptr, nullptr, useful, useful, bytes, useful};
    if (g_prof.on) {
      rec.a = g_prof.get();
      rec.b = g_prof.get();
      if (!rec.a || !rec.b || hipEventRecord(rec.a, stream) != hipSuccess)
        return fail(DION_E_HIP, "profiling event failed");
    }
    const int e = fn();
    if (e != DION_OK) return e;
    if (g_prof.on) {
      if (hipEventRecord(rec.b, stream) != hipSuccess) return fail(DION_E_HIP, "profiling event failed");
      g_prof.recs.push_back(rec);
    }
    return DION_OK;
  };
  // kernel instance names as profilers print them
  auto gemm_name = [](bool ta, bool tb, bool f16) {
    // <A layout, B layout, F16>: layout 0 r contiguous, 1 k contiguous, 2 split
    static const char* names[8] = {
        "dion::k_lr_gemm<1, 0, false>", "dion::k_lr_gemm<1, 1, false>",
        "dion::k_lr_gemm<0, 0, false>", "dion::k_lr_gemm<0, 1, false>",
        "dion::k_lr_gemm<1, 0, true>",  "dion::k_lr_gemm<1, 1, true>",
        "dion::k_lr_gemm<0, 0, true>",  "dion::k_lr_gemm<0, 1, true>"};
    return names[(f16 ? 4 : 0) + (ta ? 2 : 0) + (tb ? 1 : 0)];
  };
  bool any_small = false, any_large = false;
  for (int i = 0; i < batch; ++i) (P.r[i] <= LR_REG_RMAX ? any_small : any_large) = true;
  double elems = 0.0;
  for (int i = 0; i < batch; ++i) elems += (double)P.R[i] * P.C[i];
  // product of one group: row-major C (m x n) = op(A) op(B) with inner dimension k;
  // sa, sb: the operands' max slots, sc: the result's (-1: none).  Two-term
  // fp16 operands (f16), or three-term bf16 ones for the power product B Q,
  // whose error the orthogonalization after it amplifies by the condition
  // number of B Q
  // withg: A is the buffer M and the operand B = fl32(M + G) (gslot >= 0:
  // raise that slot with its largest |value|)
  auto gprod = [&](const char* name, const LrGroup& g, bool ta, bool tb, bool f16, int m, int n, int k, float alpha,
                   int A, int B, int Cm, int sa, int sb, int sc, int out_fmt, bool withg, int gslot,
                   double bytes_each) -> int {
    const double cnt = (double)g.mats.size();
    return phase(name, gemm_name(ta, tb, f16), 2.0 * m * n * k * cnt, bytes_each * cnt, [&]() {
      launch_lr_gemm(ta, tb, f16, m, n, k, alpha, (const float* const*)arrays(g, A), (const float* const*)arrays(g, B),
                     (void* const*)arrays(g, Cm), (unsigned* const*)arrays(g, LP_AM), sa, sb, sc, out_fmt,
                     withg ? (const uint16_t* const*)arrays(g, LP_G) : nullptr, grad_dtype, gslot,
                     (int)g.mats.size(), stream);
      return DION_OK;
    });
  };

  // split copies of a group's rows x r operand (fp16 hi and lo rows of ldp =
  // r rounded up to 32, rows padded to a multiple of 128)
  auto pad128 = [](int x) { return (x + 127) / 128 * 128; };
  auto gsplit = [&](const LrGroup& g, int src, int dst, int rows, int slot) -> int {
    const int ldp = (g.r + 31) / 32 * 32;
    const double cnt = (double)g.mats.size();
    return phase("lr_split", "dion::k_lr_split16", 0.0, cnt * (4.0 * rows * g.r + 4.0 * pad128(rows) * ldp), [&]() {
      launch_lr_split16((const float* const*)arrays(g, src), (uint16_t* const*)arrays(g, dst), rows, pad128(rows), g.r,
                        ldp, (unsigned* const*)arrays(g, LP_AM), slot, (int)g.mats.size(), stream);
      return DION_OK;
    });
  };
  // C (R x C) = alpha P Z^T + beta C from the split P and Z (C x r), inner dimension r
  auto gprod_split = [&](const char* name, const LrGroup& g, float alpha, int Z, float beta_, int Cm, int sz,
                         int out_fmt, bool withg, double bytes_each) -> int {
    const int ldp = (g.r + 31) / 32 * 32;
    const double cnt = (double)g.mats.size();
    return phase(name, out_fmt == 0 ? "dion::k_lr_gemm_dma<1>" : "dion::k_lr_gemm_dma<2>", 2.0 * g.R * g.C * g.r * cnt,
                 bytes_each * cnt, [&]() {
      launch_lr_gemm_split(g.R, g.C, g.r, ldp, pad128(g.R), pad128(g.C), alpha, (const uint16_t* const*)arrays(g, LP_XS),
                           (const uint16_t* const*)arrays(g, Z), beta_, (void* const*)arrays(g, Cm),
                           (unsigned* const*)arrays(g, LP_AM), LS_F2, sz, -1, out_fmt,
                           withg ? (const uint16_t* const*)arrays(g, LP_G) : nullptr, grad_dtype,
                           (int)g.mats.size(), stream);
      return DION_OK;
    });
  };
  const double gsz = (double)dtype_bytes(grad_dtype);
  double cr_all = 0.0;
  for (int i = 0; i < batch; ++i) cr_all += (double)P.C[i] * P.r[i];
  // With 16-bit gradients the buffer B = fl32(M + G) is never stored: the
  // power product, the right factor and the buffer update form it as they
  // read M and G (the power product also raising B's max slot), and M takes
  // the updated buffer in the last of them.  fp32 gradients take a pass that
  // stores B into M first.
  const bool fused = grad_dtype != DION_FP32;
  if (!fused) {
    if ((rc = phase("lr_accumulate", "dion::k_lr_accumulate", 0.0, elems * (8.0 + gsz), [&]() {
           launch_lr_accumulate(d_descs, nmat, P.blocks, grad_dtype, (float*)(ws + P.off_blockmax), stream);
           return DION_OK;
         })) != DION_OK) return rc;
    if ((rc = phase("lr_absmax", "dion::k_lr_absmax", 0.0, 4.0 * P.blocks, [&]() {
           launch_lr_absmax(d_descs, nmat, (const float*)(ws + P.off_blockmax), stream);
           return DION_OK;
         })) != DION_OK) return rc;
  }
  const double bsz = fused ? 4.0 + gsz : 4.0;   // bytes read per element of B
  for (const LrGroup& g : P.groups)   // Y = B Q
    if ((rc = gprod("lr_power", g, false, false, false, g.R, g.r, g.C, 1.f, LP_M, LP_Q, LP_Y, LS_B, LS_B, LS_Y, 1,
                    fused, fused ? LS_B : -1,
                    bsz * g.R * g.C + 4.0 * ((double)g.C * g.r + (double)g.R * g.r))) != DION_OK) return rc;
  // shifted CholeskyQR3 of F (rows x r): F -> dst -> tmp -> dst (tmp may be F).
  // The first pass factors S + 1e-3 max_i S_ii I: an ill-conditioned F (its
  // fp32 Gram matrix losing the small directions to rounding) then still
  // gives a factor of condition at most about 30, which two plain passes
  // (CholeskyQR2) make orthonormal to working precision; a well-conditioned F
  // is unaffected (shifted CholeskyQR, Fukaya, Kannan, Nakatsukasa, Yamamoto
  // and Yanagisawa, SIAM J. Sci. Comput. 2020, with a practical shift in
  // place of their worst-case one)
  constexpr float kShift = 1e-3f;
  // F's max slot is s_in; pass p writes its factor L_p^-1 into slot s_l + p
  // and its result into slot s_out + p
  auto cholqr3 = [&](int F, int tmp, int dst, bool rows_are_R, int s_in, int s_l, int s_out) -> int {
    const int from[3] = {F, dst, tmp}, to[3] = {dst, tmp, dst};
    for (int pass = 0; pass < 3; ++pass) {
      const int s_from = pass == 0 ? s_in : s_out + pass - 1;
      for (const LrGroup& g : P.groups) {   // S = F^T F, K split: lower tiles of each chunk's partial
        const int rows = rows_are_R ? g.R : g.C;
        const double cnt = (double)g.mats.size(), parts = (rows + LR_GRAM_CHUNK - 1) / LR_GRAM_CHUNK;
        const int e = phase("lr_orth", "dion::k_lr_gemm<0, 0, true>", 2.0 * g.r * g.r * rows * cnt,
                            cnt * 4.0 * ((double)rows * g.r + parts * g.r * g.r), [&]() {
                              launch_lr_gram(rows, g.r, (const float* const*)arrays(g, from[pass]), arrays(g, LP_S),
                                             (unsigned* const*)arrays(g, LP_AM), s_from, (int)g.mats.size(), stream);
                              return DION_OK;
                            });
        if (e != DION_OK) return e;
      }
      double rr = 0.0;
      for (int i = 0; i < batch; ++i) rr += (double)P.r[i] * P.r[i];
      int e = phase("lr_cholinv", "dion::k_lr_cholinv", 0.0, rr * 8.0, [&]() {
        launch_lr_cholinv(d_descs, nmat, any_small, any_large, rows_are_R, pass == 0 ? kShift : 0.f, s_l + pass,
                          stream);
        return DION_OK;
      });
      if (e != DION_OK) return e;
      for (const LrGroup& g : P.groups) {
        const int rows = rows_are_R ? g.R : g.C;
        e = gprod("lr_orth", g, false, true, true, rows, g.r, g.r, 1.f, from[pass], LP_L, to[pass], s_from, s_l + pass,
                  s_out + pass, 1, false, -1, 4.0 * (2.0 * rows * g.r + (double)g.r * g.r));
        if (e != DION_OK) return e;
      }
    }
    return DION_OK;
  };
  if ((rc = cholqr3(LP_Y, LP_Y, LP_X, true, LS_Y, LS_L0, LS_F0)) != DION_OK) return rc;   // P = orth(Y), in X
  for (const LrGroup& g : P.groups)   // the split P, for the buffer update and the update
    if ((rc = gsplit(g, LP_X, LP_XS, g.R, LS_F2)) != DION_OK) return rc;
  for (const LrGroup& g : P.groups)   // W = B^T P
    if ((rc = gprod("lr_right", g, true, false, true, g.C, g.r, g.R, 1.f, LP_M, LP_X, LP_W, LS_B, LS_F2, LS_W, 1,
                    fused, -1, bsz * g.R * g.C + 4.0 * ((double)g.R * g.r + (double)g.C * g.r))) != DION_OK) return rc;
  for (const LrGroup& g : P.groups)
    if ((rc = gsplit(g, LP_W, LP_WS, g.C, LS_W)) != DION_OK) return rc;
  for (const LrGroup& g : P.groups)   // M = B - beta P W^T
    if ((rc = gprod_split("lr_feedback", g, -beta, LP_WS, 1.f, LP_M, LS_W, 1, fused,
                          (bsz + 4.0) * g.R * g.C + 4.0 * ((double)g.R * g.r + (double)g.C * g.r))) != DION_OK) return rc;
  if (mode == DION_LOWRANK_QR) {
    if ((rc = cholqr3(LP_W, LP_W2, LP_Q, false, LS_W, LS_L3, LS_G0)) != DION_OK) return rc;
  } else {
    if ((rc = phase("lr_colnorm", "dion::k_lr_colnorm", 0.0, cr_all * 8.0, [&]() {
           launch_lr_colnorm(d_descs, nmat, stream);
           return DION_OK;
         })) != DION_OK) return rc;
  }
  for (const LrGroup& g : P.groups)
    if ((rc = gsplit(g, LP_Q, LP_QS, g.C, LS_G2)) != DION_OK) return rc;
  const double ob = (double)dtype_bytes(out_dtype);
  for (const LrGroup& g : P.groups)   // D = P Q^T, in the output dtype
    if ((rc = gprod_split("lr_update", g, 1.f, LP_QS, 0.f, LP_D, LS_G2, out_dtype, false,
                          ob * g.R * g.C + 4.0 * ((double)g.R * g.r + (double)g.C * g.r))) != DION_OK) return rc;
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail("kernel launch", e);
  return DION_OK;
}

// ------------------------------------------------ allocation-free scratch
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops): dion_orth_batched_noalloc runs the plan of
// dion_orth_batched in this fixed array instead of a caller's workspace.  Each
// device that the library runs on holds its own copy until the process ends.
// In host code `scratch` only names the array; its device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[DION_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices) return fail(DION_E_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail("hipGetSymbolAddress of the scratch array", e);
    if (!ptr || ((uintptr_t)ptr & 255) != 0) return fail(DION_E_HIP, "scratch array address is not 256-byte aligned");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DION_OK;
}

}  // namespace

extern "C" {

size_t dion_workspace_size(const dion_shape* shapes, int32_t batch, int32_t dtype, const dion_ns_params* p) {
  Params prm;
  if (parse_params(p, dtype, false, prm)) return 0;
  Plan P;
  if (build_plan(shapes, batch, dtype, prm, false, P)) return 0;
  size_t need = P.total;
  if (dtype == DION_FP32 && p->precision != DION_PREC_FP64) {  // may also serve dion_rowsubset_step
    Params ps;
    Plan Q;
    if (parse_params(p, DION_FP32, true, ps) == DION_OK && build_plan(shapes, batch, DION_FP32, ps, true, Q) == DION_OK)
      need = std::max(need, Q.total);
  }
  return need;
}

size_t dion_workspace_size_capped(const dion_shape* shapes, int32_t batch, int32_t dtype, const dion_ns_params* p,
                                  size_t cap) {
  Params prm;
  if (parse_params(p, dtype, false, prm)) return 0;
  std::vector<Wave> waves;
  size_t need = 0;
  if (plan_waves(shapes, batch, dtype, prm, false, 2, cap, waves, need)) return 0;
  if (dtype == DION_FP32 && p->precision != DION_PREC_FP64) {  // may also serve dion_rowsubset_step
    Params ps;
    size_t need2 = 0;
    if (parse_params(p, DION_FP32, true, ps) == DION_OK &&
        plan_waves(shapes, batch, DION_FP32, ps, true, 4, cap, waves, need2) == DION_OK)
      need = std::max(need, need2);
  }
  return need;
}

int dion_orth_batched(const void* const* M, void* const* out, const dion_shape* shapes, int32_t batch,
                      int32_t dtype, const dion_ns_params* p, int32_t* sel_idx, void* workspace,
                      size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  Params prm;
  int rc = parse_params(p, dtype, false, prm);
  if (rc) return rc;
  std::vector<Wave> waves;
  size_t need = 0;
  rc = plan_waves(shapes, batch, dtype, prm, false, 2, workspace ? workspace_bytes : (size_t)-1, waves, need);
  if (rc) return rc;
  const size_t es = dtype_bytes(dtype);
  rc = check_ptrs(M, out, shapes, batch, es, es);
  if (rc) return rc;
  for (const Wave& w : waves) {
    rc = run(w.plan, M + w.i0, out + w.i0, nullptr, w.n, dtype, dtype, 0.f, false, sel_idx ? sel_idx + w.sel0 : nullptr,
             workspace, workspace_bytes, (hipStream_t)stream);
    if (rc) return rc;
  }
  return DION_OK;
}

int dion_orth_batched_noalloc(const void* const* M, void* const* out, const dion_shape* shapes, int32_t batch,
                              int32_t dtype, const dion_ns_params* p, int32_t* sel_idx, void* stream) {
  g_last_error.clear();
  Params prm;
  int rc = parse_params(p, dtype, false, prm);
  if (rc) return rc;
  Plan P;
  rc = build_plan(shapes, batch, dtype, prm, false, P);
  if (rc) return rc;
  if (P.total > (size_t)DION_NOALLOC_SCRATCH_BYTES)
    return fail(DION_E_WORKSPACE, "this batch needs " + std::to_string(P.total) +
                                      " bytes of scratch; dion_orth_batched_noalloc holds " +
                                      std::to_string((size_t)DION_NOALLOC_SCRATCH_BYTES) +
                                      " (use dion_orth_batched with a workspace)");
  const size_t es = dtype_bytes(dtype);
  rc = check_ptrs(M, out, shapes, batch, es, es);
  if (rc) return rc;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  return run(P, M, out, nullptr, batch, dtype, dtype, 0.f, false, sel_idx, ws, (size_t)DION_NOALLOC_SCRATCH_BYTES,
             (hipStream_t)stream, nullptr, nullptr, nullptr, true);
}

int dion_orth_batched_simple(const void* const* M, void* const* out, const dion_shape* shapes, int32_t batch,
                             int32_t dtype, const float* ns_coeffs, int32_t n_iter, int32_t restart_every,
                             float safety, float row_frac, void* workspace, size_t workspace_bytes,
                             void* stream) {
  dion_ns_params p{};
  p.ns_coeffs = ns_coeffs;
  p.n_coeff_sets = 1;
  p.n_iter = n_iter;
  p.restart_every = restart_every;
  p.restart_mask = 0;
  p.safety = safety;
  p.row_frac = row_frac;
  p.precision = DION_PREC_AUTO;
  return dion_orth_batched(M, out, shapes, batch, dtype, &p, nullptr, workspace, workspace_bytes, stream);
}

int dion_rowsubset_step(float* const* E, const void* const* grad, void* const* out, const dion_shape* shapes,
                        int32_t batch, int32_t grad_dtype, float beta, const dion_ns_params* p, int32_t* sel_idx,
                        void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (grad_dtype != DION_BF16 && grad_dtype != DION_FP32) return fail(DION_E_INVAL, "unknown grad dtype");
  if (!std::isfinite(beta)) return fail(DION_E_INVAL, "beta must be finite");
  Params prm;
  int rc = parse_params(p, DION_FP32, true, prm);
  if (rc) return rc;
  std::vector<Wave> waves;
  size_t need = 0;
  rc = plan_waves(shapes, batch, DION_FP32, prm, true, grad_dtype == DION_BF16 ? 2 : 4,
                  workspace ? workspace_bytes : (size_t)-1, waves, need);
  if (rc) return rc;
  if (!E || !grad) return fail(DION_E_INVAL, "E or grad pointer array is NULL");
  for (int i = 0; i < batch; ++i)
    if (!E[i] || !grad[i]) return fail(DION_E_INVAL, "matrix " + std::to_string(i) + " has a NULL pointer");
  rc = check_ptrs((const void* const*)E, out, shapes, batch, 4, 2);
  if (rc) return rc;
  rc = check_ptrs(grad, out, shapes, batch, grad_dtype == DION_BF16 ? 2 : 4, 2);
  if (rc) return rc;
  for (const Wave& w : waves) {
    rc = run(w.plan, (const void* const*)(E + w.i0), out + w.i0, grad + w.i0, w.n, DION_FP32, grad_dtype, beta, true,
             sel_idx ? sel_idx + w.sel0 : nullptr, workspace, workspace_bytes, (hipStream_t)stream);
    if (rc) return rc;
  }
  return DION_OK;
}

size_t dion_phase_workspace_size(int32_t phase, const dion_shape* shapes, int32_t batch, int32_t dtype,
                                 int32_t precision, float row_frac) {
  if (phase < PH_KEYS || phase > PH_APPLY) return 0;
  static const float kOne[3] = {1.f, 0.f, 0.f};
  Plan P;
  const int dt = phase == PH_POLY ? DION_FP32 : dtype;
  if (build_phase_plan(phase, shapes, batch, dt, precision, phase == PH_KEYS ? row_frac : 1.0, kOne, P)) return 0;
  return P.total;
}

int dion_rowkeys_topk_batched(const void* const* M, const dion_shape* shapes, int32_t batch, int32_t dtype,
                              float row_frac, double* keys, int32_t* sel_idx, void* workspace,
                              size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  Plan P;
  int rc = build_phase_plan(PH_KEYS, shapes, batch, dtype, DION_PREC_MFMA16, row_frac, nullptr, P);
  if (rc) return rc;
  if (!M) return fail(DION_E_INVAL, "matrix pointer array is NULL");
  for (int i = 0; i < batch; ++i)
    if (!M[i]) return fail(DION_E_INVAL, "matrix " + std::to_string(i) + " has a NULL pointer");
  return run(P, M, nullptr, nullptr, batch, dtype, dtype, 0.f, false, sel_idx, workspace, workspace_bytes,
             (hipStream_t)stream, nullptr, keys);
}

int dion_syrk_batched(const void* const* X, float* const* G, const dion_shape* shapes, int32_t batch,
                      int32_t dtype, int32_t precision, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  Plan P;
  int rc = build_phase_plan(PH_SYRK, shapes, batch, dtype, precision, 1.0, nullptr, P);
  if (rc) return rc;
  if (!X || !G) return fail(DION_E_INVAL, "pointer arrays are NULL");
  std::vector<dion_shape> gs(batch);
  for (int i = 0; i < batch; ++i) {
    if (!X[i] || !G[i]) return fail(DION_E_INVAL, "matrix " + std::to_string(i) + " has a NULL pointer");
    gs[i] = {P.mats[i].m, P.mats[i].m};
  }
  const size_t es = dtype_bytes(dtype);
  for (int i = 0; i < batch; ++i)
    for (int j = 0; j < batch; ++j)
      if (overlaps(G[i], (size_t)gs[i].rows * gs[i].cols * 4, X[j], (size_t)shapes[j].rows * shapes[j].cols * es))
        return fail(DION_E_INVAL, "G must not overlap the inputs");
  return run(P, X, (void* const*)G, nullptr, batch, dtype, dtype, 0.f, false, nullptr, workspace, workspace_bytes,
             (hipStream_t)stream);
}

int dion_sympoly_batched(const float* const* G, float* const* Pout, const int32_t* m, int32_t batch,
                         const float* coeffs, int32_t precision, void* workspace, size_t workspace_bytes,
                         void* stream) {
  g_last_error.clear();
  if (!m) return fail(DION_E_INVAL, "m is NULL");
  if (batch < 1) return fail(DION_E_INVAL, "batch must be >= 1");
  const float* co = coeffs ? coeffs : kQuintic;
  if (!std::isfinite(co[0]) || !std::isfinite(co[1]) || !std::isfinite(co[2]))
    return fail(DION_E_INVAL, "coefficients must be finite");
  std::vector<dion_shape> shapes(batch);
  for (int i = 0; i < batch; ++i) shapes[i] = {m[i], m[i]};
  Plan P;
  int rc = build_phase_plan(PH_POLY, shapes.data(), batch, DION_FP32, precision, 1.0, co, P);
  if (rc) return rc;
  if (!G || !Pout) return fail(DION_E_INVAL, "pointer arrays are NULL");
  for (int i = 0; i < batch; ++i)
    if (!G[i] || !Pout[i]) return fail(DION_E_INVAL, "matrix " + std::to_string(i) + " has a NULL pointer");
  rc = check_ptrs((const void* const*)G, (void* const*)Pout, shapes.data(), batch, 4, 4);
  if (rc) return rc;
  return run(P, (const void* const*)G, (void* const*)Pout, nullptr, batch, DION_FP32, DION_FP32, 0.f, false,
             nullptr, workspace, workspace_bytes, (hipStream_t)stream);
}

int dion_apply_batched(const float* const* Q, const void* const* X, void* const* Y, const dion_shape* shapes,
                       int32_t batch, int32_t dtype, int32_t precision, void* workspace, size_t workspace_bytes,
                       void* stream) {
  g_last_error.clear();
  Plan P;
  int rc = build_phase_plan(PH_APPLY, shapes, batch, dtype, precision, 1.0, nullptr, P);
  if (rc) return rc;
  if (!Q || !X || !Y) return fail(DION_E_INVAL, "pointer arrays are NULL");
  for (int i = 0; i < batch; ++i)
    if (!Q[i]) return fail(DION_E_INVAL, "matrix " + std::to_string(i) + " has a NULL Q pointer");
  const size_t es = dtype_bytes(dtype);
  rc = check_ptrs(X, Y, shapes, batch, es, es);
  if (rc) return rc;
  for (int i = 0; i < batch; ++i)
    for (int j = 0; j < batch; ++j)
      if (overlaps(Y[i], (size_t)shapes[i].rows * shapes[i].cols * es, Q[j],
                   (size_t)P.mats[j].m * P.mats[j].m * 4))
        return fail(DION_E_INVAL, "Y must not overlap the inputs");
  return run(P, X, Y, nullptr, batch, dtype, dtype, 0.f, false, nullptr, workspace, workspace_bytes,
             (hipStream_t)stream, (const void* const*)Q);
}

int dion_rowsubset_step_update(float* const* E, const void* const* grad, void* const* W,
                               const dion_shape* shapes, int32_t batch, int32_t grad_dtype, int32_t w_dtype,
                               float beta, const float* alpha, float weight_decay, const dion_ns_params* p,
                               int32_t* sel_idx, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (grad_dtype != DION_BF16 && grad_dtype != DION_FP32) return fail(DION_E_INVAL, "unknown grad dtype");
  if (w_dtype != DION_BF16 && w_dtype != DION_FP32) return fail(DION_E_INVAL, "unknown weight dtype");
  if (!std::isfinite(beta)) return fail(DION_E_INVAL, "beta must be finite");
  if (!std::isfinite(weight_decay)) return fail(DION_E_INVAL, "weight_decay must be finite");
  if (!alpha) return fail(DION_E_INVAL, "alpha is NULL");
  for (int i = 0; i < batch; ++i)
    if (!std::isfinite(alpha[i])) return fail(DION_E_INVAL, "alpha must be finite");
  Params prm;
  int rc = parse_params(p, DION_FP32, true, prm);
  if (rc) return rc;
  std::vector<Wave> waves;
  size_t need = 0;
  rc = plan_waves(shapes, batch, DION_FP32, prm, true, grad_dtype == DION_BF16 ? 2 : 4,
                  workspace ? workspace_bytes : (size_t)-1, waves, need);
  if (rc) return rc;
  if (!E || !grad || !W) return fail(DION_E_INVAL, "E, grad or W pointer array is NULL");
  for (int i = 0; i < batch; ++i)
    if (!E[i] || !grad[i] || !W[i]) return fail(DION_E_INVAL, "matrix " + std::to_string(i) + " has a NULL pointer");
  const size_t wes = w_dtype == DION_BF16 ? 2 : 4;
  rc = check_ptrs((const void* const*)E, W, shapes, batch, 4, wes);
  if (rc) return rc;
  rc = check_ptrs(grad, W, shapes, batch, grad_dtype == DION_BF16 ? 2 : 4, wes);
  if (rc) return rc;
  // the final apply updates W in its epilogue; rows left out by the selection
  // are updated with the raw momentum by a pass of their own
  for (Wave& w : waves) {
    make_update(w.plan, w_dtype, weight_decay);
    rc = run(w.plan, (const void* const*)(E + w.i0), W + w.i0, grad + w.i0, w.n, DION_FP32, grad_dtype, beta, true,
             sel_idx ? sel_idx + w.sel0 : nullptr, workspace, workspace_bytes, (hipStream_t)stream, nullptr, nullptr,
             alpha + w.i0);
    if (rc) return rc;
  }
  return DION_OK;
}

double dion_useful_flops(const dion_shape* shapes, int32_t batch, const dion_ns_params* p) {
  Params prm;
  if (!shapes || batch < 1 || parse_params(p, DION_BF16, false, prm)) return 0.0;
  const int K = (int)prm.a.size();
  std::vector<int> seg;
  int L = 0;
  for (int k = 1; k <= K; ++k) {
    ++L;
    if (k == K || prm.restart[k - 1]) { seg.push_back(L); L = 0; }
  }
  double total = 0.0;
  for (int i = 0; i < batch; ++i) {
    const int k = selected_count(shapes[i].rows, prm.row_frac);
    const double m = std::min(k, shapes[i].cols), n = std::max(k, shapes[i].cols);
    for (int l : seg) total += n * m * (m + 1) + 2.0 * m * m * n + (4.0 * l - 3.0) * m * m * (m + 1);
  }
  return total;
}

int32_t dion_selected_rows(int32_t rows, float row_frac) {
  if (rows < 1 || !(row_frac > 0.f && row_frac <= 1.f)) return 0;
  return selected_count(rows, row_frac);
}

int dion_restart_points(const dion_ns_params* p, int32_t* after, int32_t cap) {
  Params P;
  const int rc = parse_params(p, DION_BF16, false, P);
  if (rc != DION_OK) return rc;
  if (cap < 0 || (cap > 0 && !after)) return fail(DION_E_INVAL, "after must hold cap entries");
  int n = 0;
  for (size_t k = 0; k < P.restart.size(); ++k)
    if (P.restart[k]) {
      if (n < cap) after[n] = (int32_t)(k + 1);
      ++n;
    }
  return n;
}

int dion_profile_enable(int enable) {
  const int prev = g_prof.on ? 1 : 0;
  g_prof.clear();
  g_prof.on = enable != 0;
  return prev;
}

int dion_profile_count(void) { return (int)g_prof.recs.size(); }

int dion_profile_get(int i, const char** name, const char** kernel, float* ms, double* useful_flops,
                     double* mfma_flops, double* bytes) {
  if (i < 0 || i >= (int)g_prof.recs.size()) return fail(DION_E_INVAL, "profile record out of range");
  const ProfRec& r = g_prof.recs[i];
  if (hipEventSynchronize(r.b) != hipSuccess) return fail(DION_E_HIP, "hipEventSynchronize failed");
  float t = 0.f;
  if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return fail(DION_E_HIP, "hipEventElapsedTime failed");
  if (name) *name = r.name;
  if (kernel) *kernel = r.kernel;
  if (ms) *ms = t;
  if (useful_flops) *useful_flops = r.useful;
  if (mfma_flops) *mfma_flops = r.raw;
  if (bytes) *bytes = r.bytes;
  return DION_OK;
}

int dion_profile_get_algorithmic(int i, double* algorithmic_flops) {
  if (i < 0 || i >= (int)g_prof.recs.size()) return fail(DION_E_INVAL, "profile record out of range");
  if (algorithmic_flops) *algorithmic_flops = g_prof.recs[i].alg;
  return DION_OK;
}

const char* dion_strerror(int status) {
  switch (status) {
    case DION_OK: return "success";
    case DION_E_INVAL: return "invalid argument";
    case DION_E_UNSUPPORTED: return "unsupported combination";
    case DION_E_WORKSPACE: return "workspace NULL, misaligned or too small";
    case DION_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* dion_last_error(void) { return g_last_error.c_str(); }

size_t dion_lowrank_workspace_size(const dion_shape* shapes, int32_t batch, int32_t rank, int32_t out_dtype) {
  LrPlan P;
  if (build_lr_plan(shapes, batch, rank, out_dtype, P) != DION_OK) return 0;
  return P.total;
}

int dion_lowrank_step(float* const* M, const void* const* grad, float* const* Q, void* const* out,
                      const dion_shape* shapes, int32_t batch, int32_t grad_dtype, int32_t out_dtype, int32_t rank,
                      float beta, int32_t mode, void* workspace, size_t workspace_bytes, void* stream) {
  LrPlan P;
  int rc = build_lr_plan(shapes, batch, rank, out_dtype, P);
  if (rc != DION_OK) return rc;
  if (!M || !grad || !Q || !out) return fail(DION_E_INVAL, "M, grad, Q and out must be non-NULL");
  if (!valid_dtype(grad_dtype)) return fail(DION_E_INVAL, "unknown gradient dtype");
  if (mode != DION_LOWRANK_QR && mode != DION_LOWRANK_COLNORM) return fail(DION_E_INVAL, "unknown mode");
  if (!std::isfinite(beta)) return fail(DION_E_INVAL, "beta must be finite");
  const size_t oes = dtype_bytes(out_dtype);
  for (int i = 0; i < batch; ++i) {
    if (!M[i] || !grad[i] || !Q[i] || !out[i]) return fail(DION_E_INVAL, "NULL matrix pointer");
    const size_t n = (size_t)P.R[i] * P.C[i];
    if (overlaps(out[i], n * oes, M[i], n * 4)) return fail(DION_E_INVAL, "out must not overlap M");
    if (overlaps(Q[i], (size_t)P.C[i] * P.r[i] * 4, M[i], n * 4)) return fail(DION_E_INVAL, "Q must not overlap M");
    // M is rewritten while the gradient is still read (by other blocks)
    if (overlaps(grad[i], n * dtype_bytes(grad_dtype), M[i], n * 4))
      return fail(DION_E_INVAL, "grad must not overlap M");
  }
  return run_lr(P, M, grad, Q, out, batch, grad_dtype, out_dtype, beta, mode, workspace, workspace_bytes,
                (hipStream_t)stream);
}

int dion_version(void) { return 100; }

}  // extern "C"
