// Autotuner ("TPSP Design" page, section 3, Profiling and fallback): after the weights load,
// each shape group (o_proj-like, down_proj-like) is profiled on synthetic device data; every
// fused candidate (each chunk size of the pipeline, and the single launch) is numerically
// checked against the conventional path before it is timed, and the token threshold compares
// the sum over groups of conventional and best fused timings (pr_threshold_from_timings).
// With both overrides set nothing is profiled.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <vector>

#include "pr_internal.h"

namespace pr {
namespace {

#define PR_HIP(call)                                                                  \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess) return fail(PR_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

#define PR_TRY(call)              \
  do {                            \
    int rc_ = (call);             \
    if (rc_ != PR_OK) return rc_; \
  } while (0)

struct DevBuf {
  void* p = nullptr;
  ~DevBuf() {
    if (p != nullptr) (void)hipFree(p);
  }
  int alloc(size_t bytes) {
    if (hipMalloc(&p, bytes) != hipSuccess) {
      (void)hipGetLastError();
      p = nullptr;
      return fail(PR_ERR_NOMEM, "tuning buffer of %zu bytes", bytes);
    }
    return PR_OK;
  }
};

float bf16f(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Candidate check against the conventional result on sampled rows.  The two paths differ by
// the bf16 rounding of y in the conventional one, and both outputs are rounded to bf16, so one
// output element may differ by one bf16 ulp (2^-7 relative) on top of the 2e-2 absolute bound
// (relative L2 <= 5e-3 as for the oracle comparison); the residual may differ per element by
// half a bf16 ulp of y (2^-8 |y|, with y = r_new - r_old) plus fp32 rounding.
bool candidate_ok(const std::vector<uint16_t>& out_f, const std::vector<uint16_t>& out_c,
                  const std::vector<float>& r_f, const std::vector<float>& r_c,
                  const std::vector<float>& r_old) {
  double d2 = 0, n2 = 0;
  for (size_t i = 0; i < out_f.size(); ++i) {
    const double a = bf16f(out_f[i]), b = bf16f(out_c[i]);
    if (!std::isfinite(a)) return false;
    d2 += (a - b) * (a - b);
    n2 += b * b;
    if (std::fabs(a - b) > 2e-2 + std::ldexp(std::max(std::fabs(a), std::fabs(b)), -7))
      return false;
  }
  if (d2 > 25e-6 * std::max(n2, 1e-30)) return false;
  for (size_t i = 0; i < r_f.size(); ++i) {
    if (!std::isfinite(r_f[i])) return false;
    const double y = std::fabs((double)r_f[i] - r_old[i]);
    const double bound = std::ldexp(y, -8) + 1e-5 * (1.0 + std::fabs((double)r_f[i]));
    if (std::fabs((double)r_f[i] - r_c[i]) > bound) return false;
  }
  return true;
}

struct Stats {
  double median = -1, p10 = 0, p90 = 0;
};

// Times every call of `calls` round-robin: each round runs each call once, bracketed by
// events on `s`; the first round warms up.  The chip's clock drifts with its power state, so
// timing one candidate after another would favour whichever ran first.
int time_round_robin(const std::vector<std::function<int()>>& calls, int rounds, hipStream_t s,
                     std::vector<Stats>* st) {
  hipEvent_t e0, e1;
  PR_HIP(hipEventCreate(&e0));
  if (const hipError_t e = hipEventCreate(&e1); e != hipSuccess) {
    (void)hipEventDestroy(e0);
    return fail(PR_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
  }
  std::vector<std::vector<double>> t(calls.size());
  int rc = PR_OK;
  for (int round = 0; round < rounds + 1 && rc == PR_OK; ++round) {
    for (size_t k = 0; k < calls.size() && rc == PR_OK; ++k) {
      (void)hipEventRecord(e0, s);
      rc = calls[k]();
      (void)hipEventRecord(e1, s);
      if (rc != PR_OK) break;
      if (hipEventSynchronize(e1) != hipSuccess) {
        rc = fail(PR_ERR_HIP, "timing sync failed");
        break;
      }
      float ms = 0;
      (void)hipEventElapsedTime(&ms, e0, e1);
      if (round > 0) t[k].push_back(ms * 1e-3);
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (rc != PR_OK) return rc;
  st->assign(calls.size(), Stats());
  for (size_t k = 0; k < calls.size(); ++k) {
    std::vector<double>& v = t[k];
    std::sort(v.begin(), v.end());
    (*st)[k].median = v[v.size() / 2];
    (*st)[k].p10 = v[v.size() / 10];
    (*st)[k].p90 = v[std::min(v.size() - 1, (v.size() * 9) / 10)];
  }
  return PR_OK;
}

}  // namespace
}  // namespace pr

using namespace pr;

extern "C" int pr_tune(const int* Ks, const int* Hs, int ngroups, int norm_kind,
                       const int* T_grid, int nT, const int* mc_cand, int nmc, int reps,
                       pr_tune_report* report, double* timings_out, void* stream) {
  clear_error();
  if (Ks == nullptr || Hs == nullptr || ngroups <= 0 || T_grid == nullptr || nT <= 0 ||
      mc_cand == nullptr || nmc <= 0 || reps <= 0)
    return fail(PR_ERR_INVALID_ARG, "bad tuning arguments");
  if (norm_kind != PR_NORM_STANDARD && norm_kind != PR_NORM_GEMMA)
    return fail(PR_ERR_INVALID_ARG, "unknown norm_kind %d", norm_kind);
  for (int i = 0; i < nT; ++i)
    if (T_grid[i] <= 0 || (i > 0 && T_grid[i] <= T_grid[i - 1]))
      return fail(PR_ERR_INVALID_ARG, "T_grid must be positive and ascending");
  for (int j = 0; j < nmc; ++j)
    if (mc_cand[j] <= 0 || mc_cand[j] > PR_MAX_MICROCHUNK)
      return fail(PR_ERR_MICROCHUNK, "candidate microchunk %d out of range", mc_cand[j]);
  int mc_ov = 0, thr_ov = 0;
  PR_TRY(read_overrides(&mc_ov, &thr_ov));
  const char* ev_mc = std::getenv("PR_MICROCHUNK_TOKENS");
  const char* ev_thr = std::getenv("PR_THRESHOLD_TOKENS");
  const bool have_mc = ev_mc != nullptr && ev_mc[0] != '\0';
  const bool have_thr = ev_thr != nullptr && ev_thr[0] != '\0';
  pr_tune_report rep_local = {INT32_MAX, T_grid[nT - 1], 0, 0};
  if (have_mc && have_thr) {
    // Both overrides: no scan and no numerical check; install them for every group.
    std::vector<int> mcs(nT, mc_ov);
    for (int g = 0; g < ngroups; ++g)
      PR_TRY(pr_set_tuning(Ks[g], Hs[g], thr_ov, T_grid[nT - 1], T_grid, mcs.data(), nT));
    rep_local.threshold_tokens = thr_ov;
    if (report != nullptr) *report = rep_local;
    return PR_OK;
  }
  std::vector<int> cands(mc_cand, mc_cand + nmc);
  if (have_mc) cands.assign(1, mc_ov);
  auto env_on = [](const char* n) {
    const char* v = std::getenv(n);
    return v != nullptr && v[0] != '\0';
  };
  const bool forced_cfg = env_on("PR_FORCE_TILE") || env_on("PR_FORCE_SPLIT") ||
                          env_on("PR_FORCE_WAVES") || env_on("PR_FORCE_STAGES") ||
                          env_on("PR_FORCE_KGROUPS") || env_on("PR_FORCE_CU_SPLIT");
  const int ncols = 3 + nmc;
  std::vector<double> t_conv(ngroups * nT, -1), t_fused(ngroups * nT, -1),
      spread(ngroups * nT, 0);
  std::vector<std::vector<int>> best_mc(ngroups, std::vector<int>(nT, cands[0]));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int Tmax = T_grid[nT - 1];
  const int gemma = norm_kind == PR_NORM_GEMMA;

  for (int g = 0; g < ngroups; ++g) {
    const int K = Ks[g], H = Hs[g];
    if (K <= 0 || H <= 0 || K % 64 || H % 64) return fail(PR_ERR_SHAPE, "group %d shape", g);
    DevBuf x, Wsrc, Wp, r0, r, w, out;
    PR_TRY(x.alloc((size_t)Tmax * K * 2));
    PR_TRY(Wsrc.alloc((size_t)K * H * 2));
    PR_TRY(Wp.alloc((size_t)K * H * 2));
    PR_TRY(r0.alloc((size_t)Tmax * H * 4));
    PR_TRY(r.alloc((size_t)Tmax * H * 4));
    PR_TRY(w.alloc((size_t)H * 4));
    PR_TRY(out.alloc((size_t)Tmax * H * 2));
    // Uniform draws scaled to the variances of the workloads: x, r ~ var 1; W ~ var 1/K.
    const float u1 = std::sqrt(3.0f);
    PR_TRY(launch_fill_bf16_hash((uint16_t*)x.p, (size_t)Tmax * K, 11u + g, u1, s));
    PR_TRY(launch_fill_bf16_hash((uint16_t*)Wsrc.p, (size_t)K * H, 23u + g, u1 / std::sqrt((float)K), s));
    PR_TRY(launch_fill_f32_hash((float*)r0.p, (size_t)Tmax * H, 37u + g, u1, 0.0f, s));
    PR_TRY(launch_fill_f32_hash((float*)w.p, (size_t)H, 41u + g, 0.17f, gemma ? 0.0f : 1.0f, s));
    PR_TRY(pr_prepare_weight((const uint16_t*)Wsrc.p, PR_WEIGHT_OUT_IN, (uint16_t*)Wp.p, K, H, s));
    PR_HIP(hipStreamSynchronize(s));

    // Rows checked at a token count T: the first min(T, 256) and the last as many (covers the
    // padded tail chunk).
    auto rows_chk_of = [](int T) { return (size_t)std::min(T, 256); };
    auto fetch = [&](int T, std::vector<uint16_t>& o, std::vector<float>& rr) -> int {
      const size_t rows_chk = rows_chk_of(T), tail0 = (size_t)T - rows_chk;
      o.resize(2 * rows_chk * H);
      rr.resize(2 * rows_chk * H);
      PR_HIP(hipMemcpyAsync(o.data(), out.p, rows_chk * H * 2, hipMemcpyDeviceToHost, s));
      PR_HIP(hipMemcpyAsync(o.data() + rows_chk * H, (uint16_t*)out.p + tail0 * H,
                            rows_chk * H * 2, hipMemcpyDeviceToHost, s));
      PR_HIP(hipMemcpyAsync(rr.data(), r.p, rows_chk * H * 4, hipMemcpyDeviceToHost, s));
      PR_HIP(hipMemcpyAsync(rr.data() + rows_chk * H, (float*)r.p + tail0 * H,
                            rows_chk * H * 4, hipMemcpyDeviceToHost, s));
      PR_HIP(hipStreamSynchronize(s));
      return PR_OK;
    };
    auto reset_r = [&](int T) -> int {
      PR_HIP(hipMemcpyAsync(r.p, r0.p, (size_t)T * H * 4, hipMemcpyDeviceToDevice, s));
      return PR_OK;
    };
    auto old_rows = [&](int T, std::vector<float>& r_old) -> int {
      const size_t rows_chk = rows_chk_of(T), tail0 = (size_t)T - rows_chk;
      r_old.resize(2 * rows_chk * H);
      PR_HIP(hipMemcpyAsync(r_old.data(), r0.p, rows_chk * H * 4, hipMemcpyDeviceToHost, s));
      PR_HIP(hipMemcpyAsync(r_old.data() + rows_chk * H, (float*)r0.p + tail0 * H,
                            rows_chk * H * 4, hipMemcpyDeviceToHost, s));
      PR_HIP(hipStreamSynchronize(s));
      return PR_OK;
    };
    auto conv_call_at = [&](int T) {
      return proj_add_rmsnorm_unfused((const uint16_t*)x.p, (const uint16_t*)Wp.p, (float*)r.p,
                                      (const float*)w.p, 1e-5f, T, K, H, norm_kind,
                                      (uint16_t*)out.p, s);
    };
    auto fused_call_at = [&](int T, int mc) {
      if (mc == PR_SINGLE_LAUNCH)
        return proj_add_rmsnorm_single_launch((const uint16_t*)x.p, (const uint16_t*)Wp.p,
                                              (float*)r.p, (const float*)w.p, 1e-5f, T, K, H,
                                              norm_kind, (uint16_t*)out.p, s);
      return proj_add_rmsnorm((const uint16_t*)x.p, (const uint16_t*)Wp.p, (float*)r.p,
                              (const float*)w.p, 1e-5f, T, K, H, mc, norm_kind, (uint16_t*)out.p,
                              s);
    };
    // The single launch is a fused candidate where some tile's columns divide H.
    pr_decision single_d;
    const bool single_ok = pr_select(1, K, H, PR_SINGLE_LAUNCH, &single_d) == PR_OK;
    clear_error();

    // Chunk projection configuration per chunk size (the CU footprint of a chunk's
    // projection): the model's best candidates, timed in the pipeline, checked like any
    // candidate.  The fastest that passes is installed for the group.
    if (!forced_cfg) {
      for (const int mc : cands) {
        if (mc > std::min(Tmax, PR_MAX_MICROCHUNK)) continue;
        const int Tc = std::min(Tmax, 4 * mc);
        struct Cand {
          double t;
          int c, split, waves;
        };
        // Candidates: the three best tile/split choices of the time model for the projection
        // alone on the GPU and the three best with half the GPU (the other stream's chunk
        // projection runs alongside in the pipeline), each with 8 and with 4 waves per
        // workgroup (the model does not separate the two).  The alone-ranking's best comes
        // first.
        auto ranking = [&](int cus) {
          std::vector<Cand> r;
          for (int c = 0; c < kNumTileCfgs; ++c)
            for (int split = 1; split <= 16 && K % (64 * split) == 0; split *= 2)
              r.push_back({model_gemm_time(std::min(mc, Tc), H, K, c, split, true, cus), c,
                           split, 8});
          std::sort(r.begin(), r.end(), [](const Cand& a, const Cand& b) { return a.t < b.t; });
          return r;
        };
        const std::vector<Cand> alone = ranking(kNumCUs), shared = ranking(kNumCUs / 2);
        std::vector<Cand> cs;
        auto add = [&](const Cand& x) {
          for (const Cand& y : cs)
            if (y.c == x.c && y.split == x.split) return;
          cs.push_back(x);
          cs.push_back({x.t, x.c, x.split, 4});
        };
        for (size_t k = 0; k < 3; ++k) {
          if (k < alone.size()) add(alone[k]);
          if (k < shared.size()) add(shared[k]);
        }
        std::vector<uint16_t> out_ref, out_try;
        std::vector<float> r_ref, r_try, r_before;
        PR_TRY(old_rows(Tc, r_before));
        PR_TRY(reset_r(Tc));
        PR_TRY(conv_call_at(Tc));
        PR_TRY(fetch(Tc, out_ref, r_ref));
        // Check every candidate, then time the ones that pass round-robin, one call each per
        // round: the chip's clock drifts with its power state, and timing candidates one after
        // another would favour whichever ran first.
        std::vector<size_t> passed;
        for (size_t k = 0; k < cs.size(); ++k) {
          PR_TRY(pr_set_chunk_config(K, H, mc, kTileBM[cs[k].c], kTileBN[cs[k].c], cs[k].split,
                                     cs[k].waves));
          PR_TRY(reset_r(Tc));
          PR_TRY(fused_call_at(Tc, mc));
          PR_TRY(fetch(Tc, out_try, r_try));
          if (candidate_ok(out_try, out_ref, r_try, r_ref, r_before)) passed.push_back(k);
        }
        std::vector<std::function<int()>> calls;
        for (size_t k : passed)
          calls.push_back([&, k, mc, Tc]() {
            const int rc = pr_set_chunk_config(K, H, mc, kTileBM[cs[k].c], kTileBN[cs[k].c],
                                               cs[k].split, cs[k].waves);
            return rc != PR_OK ? rc : fused_call_at(Tc, mc);
          });
        std::vector<Stats> st;
        if (!calls.empty()) PR_TRY(time_round_robin(calls, std::max(reps, 7), s, &st));
        double best_t = -1, first_t = -1;
        int best_k = -1;
        for (size_t n = 0; n < passed.size(); ++n) {
          const size_t k = passed[n];
          const double med = st[n].median;
          if (k == 0) first_t = med;
          if (best_t < 0 || med < best_t) {
            best_t = med;
            best_k = (int)k;
          }
        }
        // The model's first choice stands unless a measured candidate beats it by more than 3%
        // (near-ties would otherwise flip with timing noise from one tuning to the next).
        if (first_t > 0 && first_t <= 1.03 * best_t) best_k = 0;
        const Cand& pick = cs[best_k >= 0 ? best_k : 0];
        PR_TRY(pr_set_chunk_config(K, H, mc, kTileBM[pick.c], kTileBN[pick.c], pick.split,
                                   pick.waves));

        // The CU split with this chunk size, tuned jointly with the chunk projection's
        // configuration (the page tunes SM-count targets together with the microchunk): the
        // ping-pong schedule with the configuration just chosen, against the partitioned
        // schedule with 32 and 64 CUs reserved for the add/norms, each with the time model's
        // two best configurations for the CUs the projections keep.  Each candidate is
        // checked, then all are timed round-robin; a partition is installed only if it beats
        // the ping-pong schedule by more than 3%.
        struct SplitCand {
          int cus, c, split, waves;
        };
        std::vector<SplitCand> sc = {{0, best_k >= 0 ? pick.c : cs[0].c, pick.split, pick.waves}};
        for (const int n : {32, 64}) {
          std::vector<Cand> rk = ranking(kNumCUs - n);
          for (size_t k = 0; k < rk.size() && k < 2; ++k) sc.push_back({n, rk[k].c, rk[k].split, 8});
        }
        auto install = [&](const SplitCand& x) -> int {
          PR_TRY(pr_set_chunk_config(K, H, mc, kTileBM[x.c], kTileBN[x.c], x.split, x.waves));
          return pr_set_cu_split(K, H, mc, x.cus);
        };
        std::vector<size_t> sc_ok;
        for (size_t k = 0; k < sc.size(); ++k) {
          PR_TRY(install(sc[k]));
          PR_TRY(reset_r(Tc));
          PR_TRY(fused_call_at(Tc, mc));
          PR_TRY(fetch(Tc, out_try, r_try));
          if (candidate_ok(out_try, out_ref, r_try, r_ref, r_before)) sc_ok.push_back(k);
        }
        std::vector<std::function<int()>> split_calls;
        for (size_t k : sc_ok)
          split_calls.push_back([&, k, mc, Tc]() {
            const int rc = install(sc[k]);
            return rc != PR_OK ? rc : fused_call_at(Tc, mc);
          });
        std::vector<Stats> sst;
        if (!split_calls.empty()) PR_TRY(time_round_robin(split_calls, std::max(reps, 7), s, &sst));
        size_t best_sc = 0;
        double t0 = -1, tb = -1;
        for (size_t n = 0; n < sc_ok.size(); ++n) {
          if (sc_ok[n] == 0) t0 = sst[n].median;
          if (tb < 0 || sst[n].median < tb) {
            tb = sst[n].median;
            best_sc = sc_ok[n];
          }
        }
        if (t0 > 0 && t0 <= 1.03 * tb) best_sc = 0;
        PR_TRY(install(sc[best_sc]));
      }
    }

    for (int i = 0; i < nT; ++i) {
      const int T = T_grid[i];
      std::vector<float> r_old;
      PR_TRY(old_rows(T, r_old));
      std::vector<uint16_t> out_c, out_f;
      std::vector<float> r_c, r_f;
      PR_TRY(reset_r(T));
      PR_TRY(conv_call_at(T));
      PR_TRY(fetch(T, out_c, r_c));
      for (int j = 0; j < nmc + 1; ++j)
        if (timings_out != nullptr) timings_out[(g * nT + i) * ncols + 2 + j] = -1;
      // Fused candidates at T: every chunk size that fits and the single launch; each is
      // checked against the conventional result, then all that pass are timed round-robin
      // with the conventional path.
      std::vector<int> fused_cands;
      for (const int mc : cands)
        if (mc <= std::min(T, PR_MAX_MICROCHUNK)) fused_cands.push_back(mc);
      if (single_ok && !have_mc) fused_cands.push_back(PR_SINGLE_LAUNCH);
      std::vector<int> passed;
      for (const int mc : fused_cands) {
        PR_TRY(reset_r(T));
        PR_TRY(fused_call_at(T, mc));
        PR_TRY(fetch(T, out_f, r_f));
        if (!candidate_ok(out_f, out_c, r_f, r_c, r_old)) {
          ++rep_local.n_rejected;
          continue;
        }
        ++rep_local.n_checked;
        passed.push_back(mc);
      }
      std::vector<std::function<int()>> calls;
      calls.push_back([&, T]() { return conv_call_at(T); });
      for (const int mc : passed) calls.push_back([&, T, mc]() { return fused_call_at(T, mc); });
      std::vector<Stats> st;
      PR_TRY(time_round_robin(calls, std::max(reps, 5), s, &st));
      t_conv[g * nT + i] = st[0].median;
      if (timings_out != nullptr) timings_out[(g * nT + i) * ncols + 0] = st[0].median;
      double best = -1, best_spread = 0;
      for (size_t k = 0; k < passed.size(); ++k) {
        const int mc = passed[k];
        const Stats& sf = st[k + 1];
        if (timings_out != nullptr) {
          for (int jj = 0; jj < nmc; ++jj)
            if (mc_cand[jj] == mc) timings_out[(g * nT + i) * ncols + 2 + jj] = sf.median;
          if (mc == PR_SINGLE_LAUNCH) timings_out[(g * nT + i) * ncols + 2 + nmc] = sf.median;
        }
        if (best < 0 || sf.median < best) {
          best = sf.median;
          best_spread = sf.p90 - sf.p10;
          best_mc[g][i] = mc;
        }
      }
      t_fused[g * nT + i] = best;
      spread[g * nT + i] = best_spread;
      if (timings_out != nullptr) timings_out[(g * nT + i) * ncols + 1] = best;
    }
  }
  int thr = INT32_MAX;
  PR_TRY(pr_threshold_from_timings(ngroups, nT, T_grid, t_conv.data(), t_fused.data(),
                                   spread.data(), &thr));
  for (int g = 0; g < ngroups; ++g)
    PR_TRY(pr_set_tuning(Ks[g], Hs[g], thr, Tmax, T_grid, best_mc[g].data(), nT));
  rep_local.threshold_tokens = thr;
  if (report != nullptr) *report = rep_local;
  return PR_OK;
}
