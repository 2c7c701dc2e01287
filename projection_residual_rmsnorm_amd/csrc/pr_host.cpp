// Host-only logic of the library: argument checks, the per-call path decision, the projection
// tile choice, the dry-run schedule of the microchunk pipeline and the token-threshold search.
// Nothing here touches a GPU, so all of it is testable on a machine without one.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <map>
#include <tuple>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "pr_internal.h"

namespace pr {

namespace {
thread_local std::string g_last_error;

struct Tuning {
  int threshold = INT32_MAX;
  int max_tokens = 0;
  std::vector<int> T_grid;
  std::vector<int> mc_for_T;
};
std::mutex g_tuning_mu;
std::map<std::pair<int, int>, Tuning> g_tuning;  // keyed by (K, H)
// Tuned projection configuration of the chunks, keyed by (K, H, microchunk).
std::map<std::tuple<int, int, int>, GemmCfg> g_chunk_cfg;

constexpr long long kMaxWeightElems = 1LL << 30;  // K*H <= 2^30 (2 GiB of bf16)
}  // namespace

bool log_enabled() {
  const char* v = std::getenv("PR_LOG");
  return v != nullptr && v[0] != '\0' && v[0] != '0';
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  if (log_enabled()) std::fprintf(stderr, "[proj_add_rmsnorm] error %d: %s\n", code, buf);
  return code;
}

void clear_error() { g_last_error.clear(); }

static int parse_env_int(const char* name, int* out) {
  *out = 0;
  const char* v = std::getenv(name);
  if (v == nullptr || v[0] == '\0') return PR_OK;
  char* end = nullptr;
  const long x = std::strtol(v, &end, 10);
  if (end == v || *end != '\0' || x < 0 || x > INT32_MAX)
    return fail(PR_ERR_INVALID_ARG, "%s=\"%s\" is not a non-negative integer", name, v);
  *out = (int)x;
  return PR_OK;
}

int read_overrides(int* mc_override, int* threshold_override) {
  int rc = parse_env_int("PR_MICROCHUNK_TOKENS", mc_override);
  if (rc != PR_OK) return rc;
  if (*mc_override > PR_MAX_MICROCHUNK)
    return fail(PR_ERR_MICROCHUNK, "PR_MICROCHUNK_TOKENS=%d exceeds the cap of %d tokens",
                *mc_override, PR_MAX_MICROCHUNK);
  return parse_env_int("PR_THRESHOLD_TOKENS", threshold_override);
}

static bool env_set(const char* name) {
  const char* v = std::getenv(name);
  return v != nullptr && v[0] != '\0';
}

// Debug override of the projection tile: PR_FORCE_TILE="BMxBN" (an instantiated tile),
// PR_FORCE_WAVES=4|8, PR_FORCE_STAGES=N (an instantiated ring depth of the tile) and
// PR_FORCE_SPLIT=S (S must divide K/64; for the single launch 1, or 2 for the pair form with
// the 256x256 tile and 8 waves).  Used by tests to reach every kernel variant.
static int apply_forced_tile(int K, GemmCfg* g) {
  const char* t = std::getenv("PR_FORCE_TILE");
  if (t != nullptr && t[0] != '\0') {
    int bm = 0, bn = 0;
    bool ok = std::sscanf(t, "%dx%d", &bm, &bn) == 2;
    bool known = bm == 192 && bn == 192;  // the single launch's 12-wave tile
    for (int c = 0; c < kNumTileCfgs; ++c) known |= (kTileBM[c] == bm && kTileBN[c] == bn);
    if (!ok || !known) return fail(PR_ERR_INVALID_ARG, "PR_FORCE_TILE=\"%s\" is not a tile", t);
    g->bm = bm;
    g->bn = bn;
  }
  const char* wv = std::getenv("PR_FORCE_WAVES");
  if (wv != nullptr && wv[0] != '\0') {
    const int waves = std::atoi(wv);
    if (waves != 4 && waves != 8 && waves != 12)
      return fail(PR_ERR_INVALID_ARG, "PR_FORCE_WAVES=%s must be 4, 8 or 12", wv);
    g->waves = waves;
  }
  const char* st = std::getenv("PR_FORCE_STAGES");
  if (st != nullptr && st[0] != '\0') {
    const int stages = std::atoi(st);
    if (stages < 2 || stages > 8)
      return fail(PR_ERR_INVALID_ARG, "PR_FORCE_STAGES=%s must be in 2..8", st);
    g->stages = stages;
  }
  // A forced tile or wave count means the one-group form unless K groups are forced as well.
  if ((t != nullptr && t[0] != '\0') || (wv != nullptr && wv[0] != '\0')) g->kgroups = 1;
  const char* kgv = std::getenv("PR_FORCE_KGROUPS");
  if (kgv != nullptr && kgv[0] != '\0') {
    const int kg = std::atoi(kgv);
    if (kg != 1 && kg != 2) return fail(PR_ERR_INVALID_ARG, "PR_FORCE_KGROUPS=%s must be 1 or 2", kgv);
    g->kgroups = kg;
  }
  const char* sp = std::getenv("PR_FORCE_SPLIT");
  if (sp != nullptr && sp[0] != '\0') {
    const int split = std::atoi(sp);
    if (split <= 0 || K % (64 * split) != 0)
      return fail(PR_ERR_INVALID_ARG, "PR_FORCE_SPLIT=%s must divide K/64 = %d", sp, K / 64);
    g->split = split;
  }
  return PR_OK;
}

// ---------------------------------------------------------------------------------------------
// Projection tile choice: a time model fitted to measured projection times on MI355X (random
// bf16 data; the fit is within a few percent on shapes from 256 x 4096 x 4096 to 32768 x 8192
// x 8192).  Under sustained MFMA load the chip is power-limited, so it delivers about R flop/s
// in total however many CUs are busy, while a CU whose neighbours idle runs up to a per-tile
// ceiling r_max (clock headroom, its own load path).  A round of `active` workgroups (one per
// CU) therefore runs each CU at min(r_max, eff * R / active).  The last, partial round is timed
// at its own size.  Output writes (bf16 y or `split` fp32 planes) cost bytes / BW_W, and the
// add/norm's read of the planes bytes / BW_R.
// ---------------------------------------------------------------------------------------------
namespace {
constexpr double kChipRate = 1.3e15;                           // R, flop/s
constexpr double kTileEff[kNumTileCfgs] = {1.0, 0.85, 0.7};    // 256x256, 256x128, 128x128
constexpr double kTileRmax[kNumTileCfgs] = {7.0e12, 4.5e12, 3.5e12};  // per CU, flop/s
constexpr double kFixedK = 64;   // per-workgroup fixed cost in K-elements (prologue, epilogue)
constexpr double kWriteBW = 6.0e12;
constexpr double kReadBW = 5.5e12;
}  // namespace

static double model_tile_time(int M, int N, int K, int bm, int bn, double eff, double rmax,
                              int split, bool fp32_out, int cus) {
  const long long units = (long long)((M + bm - 1) / bm) * ((N + bn - 1) / bn) * split;
  const long long full = units / cus, rem = units % cus;
  const double tile_flops = 2.0 * bm * bn * ((double)K / split + kFixedK);
  const double chip = kChipRate * cus / kNumCUs;  // the share of the chip's rate
  auto round_t = [&](long long active) {
    return tile_flops / std::min(rmax, eff * chip / (double)active);
  };
  double t = (double)full * round_t(cus) + (rem > 0 ? round_t(rem) : 0.0);
  const bool planes = fp32_out || split > 1;
  const double y_bytes = (planes ? 4.0 * split : 2.0) * M * (double)N;
  return t + y_bytes / kWriteBW + y_bytes / kReadBW;
}

double model_gemm_time(int M, int N, int K, int c, int split, bool fp32_out, int cus) {
  return model_tile_time(M, N, K, kTileBM[c], kTileBN[c], kTileEff[c], kTileRmax[c], split,
                         fp32_out, cus);
}

GemmCfg choose_gemm(int M, int N, int K, bool fp32_out, int cus) {
  GemmCfg best;
  best.waves = 8;
  double best_t = std::numeric_limits<double>::infinity();
  for (int c = 0; c < kNumTileCfgs; ++c) {
    for (int split = 1; split <= 16; split *= 2) {
      if (K % (64 * split) != 0) break;
      const double t = model_gemm_time(M, N, K, c, split, fp32_out, cus);
      if (t < best_t * 0.999) {
        best_t = t;
        best.bm = kTileBM[c];
        best.bn = kTileBN[c];
        best.split = split;
      }
    }
  }
  return best;
}

// One fp32 output plane (no K split): the modelled fastest tile with split 1.
GemmCfg choose_gemm_unsplit(int M, int N, int K) {
  GemmCfg best;
  best.waves = 8;
  double best_t = std::numeric_limits<double>::infinity();
  for (int c = 0; c < kNumTileCfgs; ++c) {
    const double t = model_gemm_time(M, N, K, c, 1, true, kNumCUs);
    if (t < best_t * 0.999) {
      best_t = t;
      best.bm = kTileBM[c];
      best.bn = kTileBN[c];
    }
  }
  return best;
}

// Tile of the single-launch path: the modelled fastest tile whose columns divide H into at most
// 64 tile columns (the kernel's row-partial limit); bm = 0 if there is none.  A 256 x 128 tile
// grid that fits in one round runs with 8 waves in two K groups (two waves per SIMD, each wave
// keeping the 128 x 64 wave tile; on 2048 x 4096 x 4096, same box, three alternating rounds:
// 0.0858-0.0861 ms against 0.0875-0.0886 ms for 4 waves and 0.0868-0.0887 ms for 8 waves in
// one group, with every tile storing its residual after the row wait).
//
// The single launch alone also has a 192 x 192 tile with 12 waves (three per SIMD, 96 x 32 wave
// tiles), for widths that are a multiple of 192 where the 256-row tiles would leave CUs idle:
// on 3000 x 3072 x 16384 it has 256 tiles against 144 of 256 x 256.  The model takes it with
// efficiency 0.9 of the chip rate and a 5.5 TFLOP/s per-CU ceiling; with_192 = false keeps to
// the tiles every form of the single launch has (the FP8 and SiluAndMul main loops).
GemmCfg choose_single(int M, int N, int K, bool with_192) {
  GemmCfg best;
  best.bm = best.bn = 0;
  best.waves = 8;
  double best_t = std::numeric_limits<double>::infinity();
  for (int c = 0; c < kNumTileCfgs; ++c) {
    if (N % kTileBN[c] != 0 || N / kTileBN[c] > 64) continue;
    const double t = model_gemm_time(M, N, K, c, 1, false, kNumCUs);
    if (t < best_t * 0.999) {
      best_t = t;
      best.bm = kTileBM[c];
      best.bn = kTileBN[c];
    }
  }
  if (with_192 && N % 192 == 0 && N / 192 <= 64 &&
      model_tile_time(M, N, K, 192, 192, 0.9, 5.5e12, 1, false, kNumCUs) < best_t * 0.999) {
    best.bm = best.bn = 192;
    best.waves = 12;
    return best;
  }
  if (best.bm == 256 && best.bn == 128 &&
      (long long)((M + 255) / 256) * (N / 128) <= kNumCUs)
    best.kgroups = 2;
  return best;
}

// A CU split of the pipeline: 0 (no partition) or a multiple of 8 CUs (whole CUs on every XCD)
// up to half the GPU.
bool valid_cu_split(int n) { return n == 0 || (n >= 8 && n <= 128 && n % 8 == 0); }

// ---------------------------------------------------------------------------------------------
// Per-call decision.
// ---------------------------------------------------------------------------------------------
int decide(int T, int K, int H, int microchunk, pr_decision* d) {
  std::memset(d, 0, sizeof(*d));
  int path = PR_PATH_CONVENTIONAL;
  int mc = 0;
  int reason = PR_REASON_UNFUSED_CALL;
  if (microchunk == PR_SINGLE_LAUNCH) {
    path = PR_PATH_SINGLE;
    reason = PR_REASON_SINGLE_CALL;
  } else if (microchunk > 0) {
    path = PR_PATH_FUSED;
    mc = microchunk;
    reason = PR_REASON_EXPLICIT;
  } else if (microchunk == 0) {
    int mc_ov = 0, thr_ov = 0;
    int rc = read_overrides(&mc_ov, &thr_ov);
    if (rc != PR_OK) return rc;
    const bool have_mc = env_set("PR_MICROCHUNK_TOKENS");
    const bool have_thr = env_set("PR_THRESHOLD_TOKENS");
    if (have_mc && mc_ov == 0)
      return fail(PR_ERR_MICROCHUNK, "PR_MICROCHUNK_TOKENS must be in 1..%d", PR_MAX_MICROCHUNK);
    if (have_mc && have_thr) {
      // Both overrides: no tuning, no numerical check.
      if (T >= thr_ov) {
        path = PR_PATH_FUSED;
        mc = mc_ov;
        reason = PR_REASON_ABOVE_THRESHOLD;
      } else {
        reason = PR_REASON_BELOW_THRESHOLD;
      }
    } else {
      Tuning tu;
      bool found = false;
      {
        std::lock_guard<std::mutex> lk(g_tuning_mu);
        auto it = g_tuning.find({K, H});
        if (it != g_tuning.end()) {
          tu = it->second;
          found = true;
        }
      }
      if (!found) {
        reason = PR_REASON_UNTUNED;
      } else if (T > tu.max_tokens) {
        return fail(PR_ERR_UNSUPPORTED,
                    "T=%d exceeds the largest tuned token count %d for K=%d H=%d", T,
                    tu.max_tokens, K, H);
      } else {
        const int thr = have_thr ? thr_ov : tu.threshold;
        if (!have_thr && tu.threshold == INT32_MAX) {
          reason = PR_REASON_INCONCLUSIVE;
        } else if (T >= thr) {
          path = PR_PATH_FUSED;
          reason = PR_REASON_ABOVE_THRESHOLD;
          if (have_mc) {
            mc = mc_ov;
          } else {
            int idx = 0;
            for (size_t i = 0; i < tu.T_grid.size(); ++i)
              if (tu.T_grid[i] <= T) idx = (int)i;
            mc = tu.mc_for_T.empty() ? std::min(T, PR_MAX_MICROCHUNK) : tu.mc_for_T[idx];
            if (mc == PR_SINGLE_LAUNCH) path = PR_PATH_SINGLE;
          }
        } else {
          reason = PR_REASON_BELOW_THRESHOLD;
        }
      }
    }
  }
  d->path = path;
  d->reason = reason;
  GemmCfg g;
  if (path == PR_PATH_FUSED) {
    const int eff = std::min(mc, std::max(T, 1));
    d->microchunk = mc;
    d->n_chunks = T > 0 ? (T + mc - 1) / mc : 0;
    d->last_valid = T > 0 ? T - (d->n_chunks - 1) * mc : 0;
    bool tuned = false;
    {
      std::lock_guard<std::mutex> lk(g_tuning_mu);
      auto it = g_chunk_cfg.find({K, H, mc});
      if (it != g_chunk_cfg.end()) {
        g = it->second;
        tuned = true;
      }
    }
    // PR_FORCE_CU_SPLIT=<n>: the CU split of every pipeline call (tests, measurements).
    const char* cs = std::getenv("PR_FORCE_CU_SPLIT");
    if (cs != nullptr && cs[0] != '\0') {
      const int n = std::atoi(cs);
      if (!valid_cu_split(n))
        return fail(PR_ERR_INVALID_ARG, "PR_FORCE_CU_SPLIT=%s must be 0 or a multiple of 8 in "
                    "8..128", cs);
      g.addnorm_cus = n;
    }
    // Untuned: the time model's configuration for the CUs the projections get.
    if (!tuned) {
      const int n = g.addnorm_cus;
      g = choose_gemm(eff, H, K, true, kNumCUs - n);
      g.addnorm_cus = n;
    }
    d->addnorm_cus = g.addnorm_cus;
  } else if (path == PR_PATH_SINGLE) {
    d->microchunk = T;
    d->n_chunks = T > 0 ? 1 : 0;
    d->last_valid = T;
    g = choose_single(std::max(T, 1), H, K, true);
    if (g.bm == 0)
      return fail(PR_ERR_SHAPE, "single launch: H=%d is not a multiple of 128 or 192 with at "
                  "most 64 tile columns", H);
  } else {
    d->microchunk = T;
    d->n_chunks = T > 0 ? 1 : 0;
    d->last_valid = T;
    g = choose_gemm(std::max(T, 1), H, K, false);
  }
  const int rc = apply_forced_tile(K, &g);
  if (rc != PR_OK) return rc;
  d->gemm_bm = g.bm;
  d->gemm_bn = g.bn;
  d->split_k = g.split;
  d->gemm_waves = g.waves;
  d->gemm_stages = g.stages;
  d->gemm_kgroups = g.kgroups;
  return PR_OK;
}

}  // namespace pr

namespace pr {
namespace {

// Checks shared by the bf16 and the FP8 region: sizes, microchunk, norm kind, eps, null
// pointers, alignment, and that the written buffers (residual, out) overlap nothing else the
// call touches.  x holds `xb` bytes per element of the projection input (4 for the merged
// gate/up output), W `eb`; `extra` lists further read-only inputs.
struct Extra {
  const void* p;
  unsigned long long bytes;
  const char* name;
};
int validate_region(const void* x, const void* W, const void* residual_inout, const void* norm_w,
                    float eps, int T, int K, int H, int microchunk, int norm_kind,
                    const void* out, unsigned xb, unsigned eb, const Extra* extra,
                    int n_extra) {
  if (T < 0 || K <= 0 || H <= 0)
    return fail(PR_ERR_INVALID_ARG, "sizes must satisfy T >= 0, K > 0, H > 0 (T=%d K=%d H=%d)",
                T, K, H);
  if (K % 64 != 0 || H % 64 != 0)
    return fail(PR_ERR_SHAPE, "K=%d and H=%d must be multiples of 64 (zero-pad at load)", K, H);
  if ((long long)K * H > kMaxWeightElems)
    return fail(PR_ERR_SHAPE, "weight K*H=%lld exceeds %lld elements", (long long)K * H,
                kMaxWeightElems);
  if ((long long)T * H > (1LL << 40) || (long long)T * K > (1LL << 40))
    return fail(PR_ERR_SHAPE, "T=%d too large", T);
  if (microchunk < -1)
    return fail(PR_ERR_MICROCHUNK, "microchunk=%d must be >= 0", microchunk);
  if (microchunk > PR_MAX_MICROCHUNK)
    return fail(PR_ERR_MICROCHUNK, "microchunk=%d exceeds the cap of %d tokens", microchunk,
                PR_MAX_MICROCHUNK);
  if (norm_kind != PR_NORM_STANDARD && norm_kind != PR_NORM_GEMMA)
    return fail(PR_ERR_INVALID_ARG, "unknown norm_kind %d", norm_kind);
  if (!(eps >= 0.0f) || std::isinf(eps))
    return fail(PR_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (T == 0) return PR_OK;
  if (x == nullptr || W == nullptr || residual_inout == nullptr || norm_w == nullptr)
    return fail(PR_ERR_INVALID_ARG, "null tensor pointer");
  // Written buffers must not overlap anything else the call touches: the residual is updated
  // in place while later chunks still read x, and out is written while x, W, the residual and
  // the norm weight are read.  Extents are the dense row-major sizes the shape arguments give.
  struct Range {
    uintptr_t lo, hi;
    const char* name;
  };
  auto range = [](const void* p, unsigned long long bytes, const char* name) {
    return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes, name};
  };
  const Range rx = range(x, (unsigned long long)xb * T * K, "x"),
              rw = range(W, (unsigned long long)eb * K * H, "W"),
              rr = range(residual_inout, 4ULL * T * H, "residual"),
              rn = range(norm_w, 4ULL * H, "norm_w");
  auto overlap = [](const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; };
  for (const Range& o : {rx, rw, rn})
    if (overlap(rr, o)) return fail(PR_ERR_INVALID_ARG, "residual overlaps %s", o.name);
  for (int i = 0; i < n_extra; ++i) {
    if (extra[i].p == nullptr) return fail(PR_ERR_INVALID_ARG, "null %s", extra[i].name);
    if ((uintptr_t)extra[i].p % 4 != 0)
      return fail(PR_ERR_INVALID_ARG, "%s must be 4-byte aligned", extra[i].name);
    if (overlap(rr, range(extra[i].p, extra[i].bytes, extra[i].name)))
      return fail(PR_ERR_INVALID_ARG, "residual overlaps %s", extra[i].name);
  }
  if (out != nullptr) {
    const Range ro = range(out, 2ULL * T * H, "out");
    for (const Range& o : {rx, rw, rr, rn})
      if (overlap(ro, o)) return fail(PR_ERR_INVALID_ARG, "out overlaps %s", o.name);
    for (int i = 0; i < n_extra; ++i)
      if (overlap(ro, range(extra[i].p, extra[i].bytes, extra[i].name)))
        return fail(PR_ERR_INVALID_ARG, "out overlaps %s", extra[i].name);
  }
  const uintptr_t a[5] = {(uintptr_t)x, (uintptr_t)W, (uintptr_t)residual_inout,
                          (uintptr_t)norm_w, (uintptr_t)out};
  for (uintptr_t p : a)
    if (p % 16 != 0) return fail(PR_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  return PR_OK;
}

}  // namespace
}  // namespace pr

using namespace pr;

extern "C" {

int pr_version(void) { return PR_VERSION; }

const char* pr_strerror(int code) {
  switch (code) {
    case PR_OK:
      return "success";
    case PR_ERR_INVALID_ARG:
      return "invalid argument";
    case PR_ERR_SHAPE:
      return "unsupported shape";
    case PR_ERR_MICROCHUNK:
      return "invalid microchunk";
    case PR_ERR_UNSUPPORTED:
      return "unsupported call";
    case PR_ERR_NOMEM:
      return "out of device memory";
    case PR_ERR_HIP:
      return "HIP error";
    default:
      return "unknown error";
  }
}

const char* pr_last_error(void) { return pr::g_last_error.c_str(); }

int pr_validate(const void* x, const void* W, const void* residual_inout, const void* norm_w,
                float eps, int T, int K, int H, int microchunk, int norm_kind, const void* out) {
  return pr::validate_region(x, W, residual_inout, norm_w, eps, T, K, H, microchunk, norm_kind,
                             out, 2, 2, nullptr, 0);
}

int pr_validate_silu(const void* gate_up, const void* W, const void* residual_inout,
                     const void* norm_w, float eps, int T, int K, int H, int norm_kind,
                     const void* out) {
  return pr::validate_region(gate_up, W, residual_inout, norm_w, eps, T, K, H, 0, norm_kind, out,
                             4, 2, nullptr, 0);
}

int pr_validate_fp8(const void* x_q, const void* x_scales, int scale_rows, const void* W_q,
                    const void* w_scale, const void* residual_inout, const void* norm_w,
                    float eps, int T, int K, int H, int norm_kind, const void* out) {
  if (scale_rows < 1) return pr::fail(PR_ERR_INVALID_ARG, "scale_rows=%d must be >= 1", scale_rows);
  const unsigned long long groups = T > 0 ? (unsigned long long)(T - 1) / scale_rows + 1 : 0;
  const pr::Extra extra[2] = {{x_scales, 4ULL * groups, "x_scales"}, {w_scale, 4, "w_scale"}};
  return pr::validate_region(x_q, W_q, residual_inout, norm_w, eps, T, K, H, 0, norm_kind, out,
                             1, 1, extra, T > 0 ? 2 : 0);
}

int pr_select(int T, int K, int H, int microchunk, pr_decision* d) {
  if (d == nullptr) return fail(PR_ERR_INVALID_ARG, "null decision");
  if (T < 0 || K <= 0 || H <= 0) return fail(PR_ERR_INVALID_ARG, "bad sizes");
  if (microchunk < PR_SINGLE_LAUNCH || microchunk > PR_MAX_MICROCHUNK)
    return fail(PR_ERR_MICROCHUNK, "microchunk=%d out of range", microchunk);
  return decide(T, K, H, microchunk, d);
}

int pr_plan(int T, int microchunk, pr_plan_op* ops, int max_ops) {
  if (T < 0 || microchunk <= 0 || microchunk > PR_MAX_MICROCHUNK)
    return fail(PR_ERR_INVALID_ARG, "pr_plan needs T >= 0 and 0 < microchunk <= %d",
                PR_MAX_MICROCHUNK);
  if (max_ops < 0 || (max_ops > 0 && ops == nullptr))
    return fail(PR_ERR_INVALID_ARG, "bad op buffer");
  int n = 0;
  auto emit = [&](int op, int stream, int chunk, int slot, int rows) {
    if (n < max_ops) ops[n] = pr_plan_op{op, stream, chunk, slot, rows};
    ++n;
  };
  if (T == 0) return 0;
  const int nc = (T + microchunk - 1) / microchunk;
  // Even chunks run on the caller's stream (0), odd chunks on the library stream (1); each
  // chunk's projection and add/norm are consecutive on one stream, so chunk c+1's projection
  // on the other stream overlaps chunk c's add/norm.  Slot c % 3 is reused by chunk c + 3,
  // which always runs on the other stream and waits for done[slot].
  auto stream_of = [](int c) { return c % 2 == 0 ? 0 : 1; };
  const int last_even = (nc - 1) % 2 == 0 ? nc - 1 : nc - 2;               // caller stream
  const int last_odd = nc >= 2 ? ((nc - 1) % 2 == 1 ? nc - 1 : nc - 2) : -1;  // library stream
  emit(PR_OP_WAIT_PREV, 0, -1, -1, 0);
  if (nc >= 2) {
    emit(PR_OP_RECORD_ENTRY, 0, -1, -1, 0);
    emit(PR_OP_WAIT_ENTRY, 1, -1, -1, 0);
  }
  auto rows_of = [&](int c) { return std::min(microchunk, T - c * microchunk); };
  auto addnorm = [&](int c) {
    emit(PR_OP_ADDNORM, stream_of(c), c, c % PR_NUM_SLOTS, rows_of(c));
    // done[slot]: waited for by chunk c + 3, by the join (the library stream's last chunk) and
    // by a next call made from another stream (the last chunk on each stream).
    if (c + PR_NUM_SLOTS < nc || c == last_even || c == last_odd)
      emit(PR_OP_RECORD_DONE, stream_of(c), c, c % PR_NUM_SLOTS, 0);
  };
  // Host order: chunk c's projection is enqueued before chunk c-1's add/norm, so that it
  // reaches the other stream while chunk c-1's projection still runs.  Each stream's own
  // order (projection, add/norm, projection, ...) is unchanged, and done[slot] of chunk c-3
  // is recorded (with that chunk's add/norm, two iterations earlier) before chunk c waits
  // for it.
  for (int c = 0; c < nc; ++c) {
    const int s = c % PR_NUM_SLOTS;
    if (c >= PR_NUM_SLOTS) emit(PR_OP_WAIT_DONE, stream_of(c), c, s, 0);
    emit(PR_OP_GEMM, stream_of(c), c, s, rows_of(c));
    if (c >= 1) addnorm(c - 1);
  }
  addnorm(nc - 1);
  if (last_odd >= 0) emit(PR_OP_JOIN, 0, last_odd, last_odd % PR_NUM_SLOTS, 0);
  return n;
}

int pr_plan_cu_split(int T, int microchunk, pr_plan_op* ops, int max_ops) {
  if (T < 0 || microchunk <= 0 || microchunk > PR_MAX_MICROCHUNK)
    return fail(PR_ERR_INVALID_ARG, "pr_plan_cu_split needs T >= 0 and 0 < microchunk <= %d",
                PR_MAX_MICROCHUNK);
  if (max_ops < 0 || (max_ops > 0 && ops == nullptr))
    return fail(PR_ERR_INVALID_ARG, "bad op buffer");
  int n = 0;
  auto emit = [&](int op, int stream, int chunk, int slot, int rows) {
    if (n < max_ops) ops[n] = pr_plan_op{op, stream, chunk, slot, rows};
    ++n;
  };
  if (T == 0) return 0;
  const int nc = (T + microchunk - 1) / microchunk;
  auto rows_of = [&](int c) { return std::min(microchunk, T - c * microchunk); };
  emit(PR_OP_WAIT_PREV, 0, -1, -1, 0);
  emit(PR_OP_RECORD_ENTRY, 0, -1, -1, 0);
  emit(PR_OP_WAIT_ENTRY, 1, -1, -1, 0);
  emit(PR_OP_WAIT_ENTRY, 2, -1, -1, 0);
  auto addnorm = [&](int c) {
    const int s = c % PR_NUM_SLOTS;
    emit(PR_OP_WAIT_READY, 2, c, s, 0);
    emit(PR_OP_ADDNORM, 2, c, s, rows_of(c));
    // done[slot]: waited for by chunk c + 3's projection and, for the last chunk, by the join
    // and by a next call made from another stream.
    if (c + PR_NUM_SLOTS < nc || c == nc - 1) emit(PR_OP_RECORD_DONE, 2, c, s, 0);
  };
  // Host order: chunk c's projection (and its slot wait) before chunk c-1's add/norm, so the
  // projection stream is fed ahead; a wait is enqueued after the record it waits for.
  for (int c = 0; c < nc; ++c) {
    const int s = c % PR_NUM_SLOTS;
    if (c >= PR_NUM_SLOTS) emit(PR_OP_WAIT_DONE, 1, c, s, 0);
    emit(PR_OP_GEMM, 1, c, s, rows_of(c));
    emit(PR_OP_RECORD_READY, 1, c, s, 0);
    if (c >= 1) addnorm(c - 1);
  }
  addnorm(nc - 1);
  emit(PR_OP_JOIN, 0, nc - 1, (nc - 1) % PR_NUM_SLOTS, 0);
  return n;
}

int pr_threshold_from_timings(int ngroups, int nT, const int* T_grid, const double* t_conv,
                              const double* t_fused, const double* spread, int* threshold) {
  if (ngroups <= 0 || nT <= 0 || T_grid == nullptr || t_conv == nullptr || t_fused == nullptr ||
      threshold == nullptr)
    return fail(PR_ERR_INVALID_ARG, "bad threshold inputs");
  for (int i = 1; i < nT; ++i)
    if (T_grid[i] <= T_grid[i - 1]) return fail(PR_ERR_INVALID_ARG, "T_grid must ascend");
  std::vector<bool> win(nT, false);
  for (int i = 0; i < nT; ++i) {
    double sc = 0, sf = 0, sp = 0;
    bool ok = true;
    for (int g = 0; g < ngroups; ++g) {
      const double c = t_conv[g * nT + i], f = t_fused[g * nT + i];
      if (!(c > 0) || !(f > 0)) ok = false;
      sc += c;
      sf += f;
      if (spread != nullptr) sp += std::max(0.0, spread[g * nT + i]);
    }
    const double margin = std::max(0.02 * sc, sp);
    win[i] = ok && (sf + margin < sc);
  }
  int thr = INT32_MAX;
  for (int i = nT - 1; i >= 0; --i) {
    if (!win[i]) break;
    thr = T_grid[i];
  }
  *threshold = thr;
  return PR_OK;
}

int pr_set_tuning(int K, int H, int threshold_tokens, int max_tokens, const int* T_grid,
                  const int* mc_for_T, int nT) {
  if (K <= 0 || H <= 0 || max_tokens < 0 || threshold_tokens < 0 || nT < 0 ||
      (nT > 0 && (T_grid == nullptr || mc_for_T == nullptr)))
    return fail(PR_ERR_INVALID_ARG, "bad tuning arguments");
  Tuning tu;
  tu.threshold = threshold_tokens;
  tu.max_tokens = max_tokens;
  for (int i = 0; i < nT; ++i) {
    if (i > 0 && T_grid[i] <= T_grid[i - 1])
      return fail(PR_ERR_INVALID_ARG, "T_grid must ascend");
    if ((mc_for_T[i] <= 0 && mc_for_T[i] != PR_SINGLE_LAUNCH) ||
        mc_for_T[i] > PR_MAX_MICROCHUNK)
      return fail(PR_ERR_MICROCHUNK, "tuned microchunk %d out of range", mc_for_T[i]);
    tu.T_grid.push_back(T_grid[i]);
    tu.mc_for_T.push_back(mc_for_T[i]);
  }
  std::lock_guard<std::mutex> lk(g_tuning_mu);
  g_tuning[{K, H}] = tu;
  return PR_OK;
}

int pr_set_chunk_config(int K, int H, int microchunk, int tile_m, int tile_n, int split_k,
                        int waves) {
  if (K <= 0 || H <= 0 || K % 64 != 0 || H % 64 != 0)
    return fail(PR_ERR_SHAPE, "K=%d and H=%d must be positive multiples of 64", K, H);
  if (microchunk <= 0 || microchunk > PR_MAX_MICROCHUNK)
    return fail(PR_ERR_MICROCHUNK, "microchunk=%d out of range", microchunk);
  bool known = false;
  for (int c = 0; c < kNumTileCfgs; ++c) known |= (kTileBM[c] == tile_m && kTileBN[c] == tile_n);
  if (!known) return fail(PR_ERR_INVALID_ARG, "no projection tile %dx%d", tile_m, tile_n);
  if (split_k <= 0 || K % (64 * split_k) != 0)
    return fail(PR_ERR_INVALID_ARG, "split_k=%d must divide K/64 = %d", split_k, K / 64);
  if (waves != 4 && waves != 8) return fail(PR_ERR_INVALID_ARG, "waves=%d must be 4 or 8", waves);
  GemmCfg g;
  g.bm = tile_m;
  g.bn = tile_n;
  g.split = split_k;
  g.waves = waves;
  std::lock_guard<std::mutex> lk(g_tuning_mu);
  auto it = g_chunk_cfg.find({K, H, microchunk});
  if (it != g_chunk_cfg.end()) g.addnorm_cus = it->second.addnorm_cus;  // kept
  g_chunk_cfg[{K, H, microchunk}] = g;
  return PR_OK;
}

int pr_set_cu_split(int K, int H, int microchunk, int addnorm_cus) {
  if (K <= 0 || H <= 0 || K % 64 != 0 || H % 64 != 0)
    return fail(PR_ERR_SHAPE, "K=%d and H=%d must be positive multiples of 64", K, H);
  if (microchunk <= 0 || microchunk > PR_MAX_MICROCHUNK)
    return fail(PR_ERR_MICROCHUNK, "microchunk=%d out of range", microchunk);
  if (!valid_cu_split(addnorm_cus))
    return fail(PR_ERR_INVALID_ARG, "addnorm_cus=%d must be 0 or a multiple of 8 in 8..128",
                addnorm_cus);
  std::lock_guard<std::mutex> lk(g_tuning_mu);
  auto it = g_chunk_cfg.find({K, H, microchunk});
  if (it == g_chunk_cfg.end())  // the model's configuration for the projections' CUs
    it = g_chunk_cfg.emplace(std::make_tuple(K, H, microchunk),
                             choose_gemm(microchunk, H, K, true, kNumCUs - addnorm_cus)).first;
  it->second.addnorm_cus = addnorm_cus;
  return PR_OK;
}

void pr_clear_tuning(void) {
  std::lock_guard<std::mutex> lk(g_tuning_mu);
  g_tuning.clear();
  g_chunk_cfg.clear();
}

// Tuning file, one record per line (tokens separated by single spaces):
//   pr_tuning 1 <library version> <device key>
//   tuning <K> <H> <threshold> <max tokens> <nT> then nT pairs <T> <chunk>
//   chunk <K> <H> <microchunk> <tile rows> <tile columns> <K split> <waves>
//   cusplit <K> <H> <microchunk> <add/norm CUs>         (after the chunk record it refines)
int pr_tuning_save(const char* path, const char* device_key) {
  if (path == nullptr) return fail(PR_ERR_INVALID_ARG, "path is NULL");
  std::string key;
  if (device_key != nullptr) {
    key = device_key;
  } else {
    const int rc = current_device_key(&key);
    if (rc != PR_OK) return rc;
  }
  if (key.empty() || key.find_first_of(" \t\n") != std::string::npos)
    return fail(PR_ERR_INVALID_ARG, "device key \"%s\" is empty or has white space", key.c_str());
  std::string text = "pr_tuning 1 " + std::to_string(PR_VERSION) + " " + key + "\n";
  {
    std::lock_guard<std::mutex> lk(g_tuning_mu);
    for (const auto& kv : g_tuning) {
      const Tuning& tu = kv.second;
      text += "tuning " + std::to_string(kv.first.first) + " " + std::to_string(kv.first.second) +
              " " + std::to_string(tu.threshold) + " " + std::to_string(tu.max_tokens) + " " +
              std::to_string(tu.T_grid.size());
      for (size_t i = 0; i < tu.T_grid.size(); ++i)
        text += " " + std::to_string(tu.T_grid[i]) + " " + std::to_string(tu.mc_for_T[i]);
      text += "\n";
    }
    for (const auto& kv : g_chunk_cfg) {
      const GemmCfg& g = kv.second;
      text += "chunk " + std::to_string(std::get<0>(kv.first)) + " " +
              std::to_string(std::get<1>(kv.first)) + " " + std::to_string(std::get<2>(kv.first)) +
              " " + std::to_string(g.bm) + " " + std::to_string(g.bn) + " " +
              std::to_string(g.split) + " " + std::to_string(g.waves) + "\n";
    }
    for (const auto& kv : g_chunk_cfg)
      if (kv.second.addnorm_cus > 0)
        text += "cusplit " + std::to_string(std::get<0>(kv.first)) + " " +
                std::to_string(std::get<1>(kv.first)) + " " +
                std::to_string(std::get<2>(kv.first)) + " " +
                std::to_string(kv.second.addnorm_cus) + "\n";
  }
  FILE* f = std::fopen(path, "w");
  if (f == nullptr) return fail(PR_ERR_INVALID_ARG, "cannot write %s", path);
  const bool ok = std::fwrite(text.data(), 1, text.size(), f) == text.size();
  if (std::fclose(f) != 0 || !ok) return fail(PR_ERR_INVALID_ARG, "cannot write %s", path);
  return PR_OK;
}

namespace {
// Whole-line integer parsing: every token must be a decimal integer in int range.
bool parse_ints(const std::vector<std::string>& tok, size_t from, std::vector<long long>* out) {
  for (size_t i = from; i < tok.size(); ++i) {
    const char* b = tok[i].c_str();
    char* e = nullptr;
    const long long v = std::strtoll(b, &e, 10);
    if (e == b || *e != '\0' || v < INT32_MIN || v > INT32_MAX) return false;
    out->push_back(v);
  }
  return true;
}
}  // namespace

int pr_tuning_load(const char* path, const char* device_key) {
  if (path == nullptr) return fail(PR_ERR_INVALID_ARG, "path is NULL");
  std::string key;
  if (device_key != nullptr) {
    key = device_key;
  } else {
    const int rc = current_device_key(&key);
    if (rc != PR_OK) return rc;
  }
  FILE* f = std::fopen(path, "r");
  if (f == nullptr) return fail(PR_ERR_INVALID_ARG, "cannot read %s", path);
  std::vector<std::vector<std::string>> lines;
  {
    std::string cur;
    std::vector<std::string> tok;
    int c;
    while ((c = std::fgetc(f)) != EOF) {
      if (c == ' ' || c == '\n') {
        if (!cur.empty()) tok.push_back(cur);
        cur.clear();
        if (c == '\n') {
          if (!tok.empty()) lines.push_back(tok);
          tok.clear();
        }
      } else {
        cur.push_back((char)c);
      }
    }
    if (!cur.empty()) tok.push_back(cur);
    if (!tok.empty()) lines.push_back(tok);
  }
  std::fclose(f);
  if (lines.empty() || lines[0].size() != 4 || lines[0][0] != "pr_tuning" || lines[0][1] != "1")
    return fail(PR_ERR_INVALID_ARG, "%s is not a tuning file of format 1", path);
  if (lines[0][2] != std::to_string(PR_VERSION))
    return fail(PR_ERR_UNSUPPORTED, "%s was written by library version %s (this is %d)", path,
                lines[0][2].c_str(), PR_VERSION);
  if (lines[0][3] != key)
    return fail(PR_ERR_UNSUPPORTED, "%s was tuned on device %s, not %s", path,
                lines[0][3].c_str(), key.c_str());
  // Install every record through the setters (which validate it); on any failure restore the
  // tables as they were, so a bad file installs nothing.
  std::map<std::pair<int, int>, Tuning> saved_tuning;
  std::map<std::tuple<int, int, int>, GemmCfg> saved_chunk;
  {
    std::lock_guard<std::mutex> lk(g_tuning_mu);
    saved_tuning = g_tuning;
    saved_chunk = g_chunk_cfg;
  }
  int rc = PR_OK;
  for (size_t ln = 1; ln < lines.size() && rc == PR_OK; ++ln) {
    const auto& tok = lines[ln];
    std::vector<long long> v;
    if (!parse_ints(tok, 1, &v)) {
      rc = fail(PR_ERR_INVALID_ARG, "%s line %zu: not a list of integers", path, ln + 1);
    } else if (tok[0] == "tuning" && v.size() >= 5 && v[4] >= 0 &&
               v.size() == 5 + 2 * (size_t)v[4]) {
      std::vector<int> Tg, mc;
      for (long long i = 0; i < v[4]; ++i) {
        Tg.push_back((int)v[5 + 2 * i]);
        mc.push_back((int)v[6 + 2 * i]);
      }
      rc = pr_set_tuning((int)v[0], (int)v[1], (int)v[2], (int)v[3], Tg.data(), mc.data(),
                         (int)v[4]);
    } else if (tok[0] == "chunk" && v.size() == 7) {
      rc = pr_set_chunk_config((int)v[0], (int)v[1], (int)v[2], (int)v[3], (int)v[4], (int)v[5],
                               (int)v[6]);
    } else if (tok[0] == "cusplit" && v.size() == 4) {
      rc = pr_set_cu_split((int)v[0], (int)v[1], (int)v[2], (int)v[3]);
    } else {
      rc = fail(PR_ERR_INVALID_ARG, "%s line %zu: unknown or malformed record", path, ln + 1);
    }
  }
  if (rc != PR_OK) {
    const std::string msg = pr_last_error();
    {
      std::lock_guard<std::mutex> lk(g_tuning_mu);
      g_tuning = saved_tuning;
      g_chunk_cfg = saved_chunk;
    }
    return fail(rc, "%s", msg.c_str());
  }
  return PR_OK;
}

}  // extern "C"
