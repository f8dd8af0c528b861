// Host-side check of the library under AddressSanitizer and UBSan (built and
// run by tests/test_host_sanitizers.py, on the CPU).  It links the planner and
// C ABI (dion_api.cpp) against no-op kernel launchers, and drives every
// host-only entry point over many shapes and parameter sets, plus the
// argument checks of the device entry points, which return before any launch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "dion.h"
#include "dion_internal.h"
#include "lowrank_internal.h"

namespace dion {
// never reached: every call below fails validation or only plans
bool launch_gemm16(int, int, int, int, bool, const GemmLaunch&, const PhaseArgs&, hipStream_t) { std::abort(); }
bool launch_gemm64(int, bool, const GemmLaunch&, const PhaseArgs&, hipStream_t) { std::abort(); }
void launch_rowkeys(int, bool, const MatDesc*, int, int64_t, double*, hipStream_t) { std::abort(); }
void launch_momentum_keys(bool, bool, const MatDesc*, int, int64_t, float, double*, int, hipStream_t) { std::abort(); }
void launch_update_unselected(bool, const MatDesc*, int, int64_t, const uint8_t*, float, bool, hipStream_t) {
  std::abort();
}
void launch_decay_selected(const MatDesc*, int, int64_t, const int*, float, hipStream_t) { std::abort(); }
void launch_select(const MatDesc*, int, const double*, uint8_t*, int*, MatScalars*, bool, hipStream_t) {
  std::abort();
}
void launch_pack(int, bool, const MatDesc*, const int*, const int*, int, int, const int*, const MatScalars*, int, bool,
                 hipStream_t) {
  std::abort();
}
void launch_transpose(const MatDesc*, const int*, const int*, int, int, int, int, hipStream_t) { std::abort(); }
void launch_copy_unselected(bool, const MatDesc*, int, int64_t, const uint8_t*, hipStream_t) { std::abort(); }
void launch_unpack(bool, const MatDesc*, const int*, int, int, int, const MatScalars*, float, bool, hipStream_t) {
  std::abort();
}
void launch_scale_combine(MatScalars*, int, hipStream_t) { std::abort(); }
void launch_upload(void*, const void*, size_t, hipStream_t) { std::abort(); }
void launch_tiny_gns(const MatDesc*, const int*, int, const MatScalars*, const int*, const double*, int, unsigned long long, int,
                     int, int, float, hipStream_t) {
  std::abort();
}
void launch_lr_accumulate(const LrDesc*, int, int64_t, int, float*, hipStream_t) { std::abort(); }
void launch_lr_absmax(const LrDesc*, int, const float*, hipStream_t) { std::abort(); }
void launch_lr_cholinv(const LrDesc*, int, bool, bool, bool, float, int, hipStream_t) { std::abort(); }
void launch_lr_gram(int, int, const float* const*, float* const*, unsigned* const*, int, int, hipStream_t) { std::abort(); }
void launch_lr_colnorm(const LrDesc*, int, hipStream_t) { std::abort(); }
void launch_lr_gemm(bool, bool, bool, int, int, int, float, const float* const*, const float* const*, void* const*,
                    unsigned* const*, int, int, int, int, const uint16_t* const*, int, int, int, hipStream_t) {
  std::abort();
}
void launch_lr_gemm_split(int, int, int, int, int, int, float, const uint16_t* const*, const uint16_t* const*, float,
                          void* const*, unsigned* const*, int, int, int, int, const uint16_t* const*, int, int,
                          hipStream_t) {
  std::abort();
}
void launch_lr_split16(const float* const*, uint16_t* const*, int, int, int, int, unsigned* const*, int, int,
                       hipStream_t) {
  std::abort();
}
}  // namespace dion

static unsigned long long rng_state = 88172645463325252ull;
static unsigned next_u() {  // xorshift64
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (unsigned)(rng_state >> 11);
}
static int pick(int lo, int hi) { return lo + (int)(next_u() % (unsigned)(hi - lo + 1)); }

int main() {
  int planned = 0;
  const int dims[] = {1, 2, 5, 63, 64, 65, 127, 255, 256, 257, 700, 1024, 1025, 4096, 14336, 28672};
  for (int it = 0; it < 400; ++it) {
    const int batch = pick(1, 12);
    std::vector<dion_shape> sh(batch);
    for (auto& s : sh) {
      s.rows = dims[pick(0, 15)];
      s.cols = dims[pick(0, 15)];
      if (it % 3 == 0) { s.rows = pick(1, 300); s.cols = pick(1, 300); }
    }
    const int K = pick(1, 12);
    std::vector<float> co(3 * K);
    for (int k = 0; k < K; ++k) { co[3 * k] = 3.4445f; co[3 * k + 1] = -4.775f; co[3 * k + 2] = 2.0315f; }
    dion_ns_params p{};
    p.ns_coeffs = it % 2 ? co.data() : nullptr;
    p.n_coeff_sets = it % 2 ? K : 1;
    p.n_iter = K;
    p.restart_every = pick(0, 3);
    p.restart_mask = it % 5 == 0 ? (unsigned)pick(0, 255) : 0u;
    p.restart_threshold = it % 7 == 0 ? 100.0f : 0.0f;
    p.safety = it % 4 == 0 ? 1.05f : 1.0f;
    p.row_frac = (const float[]){1.0f, 0.5f, 0.25f, 0.125f, 1.0f / 37}[pick(0, 4)];
    p.precision = pick(0, 2);
    p.ef_carry = pick(0, 1);
    p.keep_schedule = pick(0, 1);
    for (int dt : {DION_BF16, DION_FP32, DION_FP16}) {
      const size_t n = dion_workspace_size(sh.data(), batch, dt, &p);
      if (n) ++planned;
    }
    (void)dion_useful_flops(sh.data(), batch, &p);
    int32_t pts[64];
    const int np = dion_restart_points(&p, pts, it % 2 ? 64 : 2);
    if (np < 0 && p.n_iter >= 1) { std::fprintf(stderr, "restart points failed\n"); return 1; }
    for (int ph = 1; ph <= 4; ++ph)
      (void)dion_phase_workspace_size(ph, sh.data(), batch, it % 3, pick(0, 2), p.row_frac);
    (void)dion_lowrank_workspace_size(sh.data(), batch, pick(1, 600), pick(0, 2));
  }
  // argument checks of the device entry points: each returns an error before any launch
  dion_shape s2[2] = {{64, 32}, {32, 64}};
  void* fake[2] = {(void*)0x10000, (void*)0x20000};
  void* alias[2] = {(void*)0x10000, (void*)0x90000};
  dion_ns_params p{};
  p.n_iter = 5;
  p.safety = 1.0f;
  p.row_frac = 1.0f;
  int bad = 0;
  bad += dion_orth_batched(nullptr, fake, s2, 2, DION_BF16, &p, nullptr, (void*)0x100000, 1 << 20, nullptr) == 0;
  bad += dion_orth_batched((const void* const*)fake, alias, s2, 2, DION_BF16, &p, nullptr, (void*)0x100000, 1 << 20,
                           nullptr) == 0;
  bad += dion_orth_batched((const void* const*)fake, fake, s2, 0, DION_BF16, &p, nullptr, (void*)0x100000, 1 << 20,
                           nullptr) == 0;
  p.n_iter = 0;
  bad += dion_orth_batched((const void* const*)fake, fake, s2, 2, DION_BF16, &p, nullptr, (void*)0x100000, 1 << 20,
                           nullptr) == 0;
  p.n_iter = 5;
  p.restart_threshold = NAN;
  bad += dion_workspace_size(s2, 2, DION_BF16, &p) != 0;
  p.restart_threshold = 0.0f;
  p.keep_schedule = 2;
  bad += dion_workspace_size(s2, 2, DION_BF16, &p) != 0;
  p.keep_schedule = 0;
  bad += dion_rowsubset_step(nullptr, nullptr, nullptr, s2, 2, DION_BF16, 0.9f, &p, nullptr, nullptr, 0, nullptr) == 0;
  bad += dion_lowrank_step(nullptr, nullptr, nullptr, nullptr, s2, 2, DION_BF16, DION_BF16, 8, 1.0f, 0, nullptr, 0,
                           nullptr) == 0;
  bad += dion_lowrank_workspace_size(s2, 2, 513, DION_BF16) != 0;
  for (int c = -5; c <= 0; ++c) (void)dion_strerror(c);
  (void)dion_last_error();
  if (bad) { std::fprintf(stderr, "%d invalid calls were accepted\n", bad); return 1; }
  std::printf("host check: %d plans, argument checks ok\n", planned);
  return planned > 0 ? 0 : 1;
}
