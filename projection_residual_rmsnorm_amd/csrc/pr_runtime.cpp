// Runtime of the library: per-device resources (one library stream, an entry event, three slot
// done events, the three-slot workspace), the microchunk pipeline executor and the
// conventional path.
//
// Pipeline ("TPSP Design" page, section 3, Microchunk pipeline): chunks alternate between the
// caller's stream and one library stream.  On its stream, chunk c's projection writes slot
// c % 3 and the chunk's residual add + RMSNorm follows it directly, while chunk c+1's
// projection runs on the other stream.  Chunk c+3 reuses the slot from the other stream and
// waits for done[slot] first.  The library stream starts after the caller's prior work (entry
// event) and the caller's stream waits for the library stream's last chunk, so the call is
// ordered on the caller's stream like a single kernel and never blocks the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <memory>
#include <mutex>
#include <vector>

#include "pr_internal.h"

namespace pr {
namespace {

constexpr int kMaxDevices = 64;

// A pair of CU-masked library streams for the CU-partitioned pipeline: `proj` may use every
// CU but the `cus` reserved ones, `addnorm` only those (spread evenly over the XCDs).
struct MaskedPair {
  int cus = 0;
  hipStream_t proj = nullptr;
  hipStream_t addnorm = nullptr;
};

struct DevCtx {
  int device = -1;
  hipStream_t sL = nullptr;  // library stream (odd chunks)
  hipEvent_t entry = nullptr;
  hipEvent_t done[PR_NUM_SLOTS] = {};
  hipEvent_t ready[PR_NUM_SLOTS] = {};  // CU-partitioned pipeline: projection -> add/norm
  MaskedPair masked;  // at most one pair per device (a process has few hardware queues)
  int cu_count = 0;
  float* slots = nullptr;  // PR_NUM_SLOTS slots of slot_elems fp32 each
  size_t slot_elems = 0;
  void* conv = nullptr;  // conventional path: bf16 y or fp32 partial planes
  size_t conv_bytes = 0;
  uint16_t* out_ws = nullptr;  // borrowed output
  size_t out_ws_bytes = 0;
  // single-launch path: row-partial slots (epoch-tagged) and the status / completion / epoch
  // words (the epoch lives on the device and advances per launch)
  void* row_slots = nullptr;
  size_t row_slots_bytes = 0;
  unsigned* sync = nullptr;
  size_t sync_bytes = 0;
  // pair form: per-tile XCD-id and ready words (epoch-tagged like the slots) and the exchange
  // regions
  void* pair_flags = nullptr;
  size_t pair_flags_bytes = 0;
  void* xbuf = nullptr;
  size_t xbuf_bytes = 0;
  // FP8 quantisation: per-row maxima
  void* row_amax = nullptr;
  size_t row_amax_bytes = 0;
  const uint16_t* last_borrowed = nullptr;
  // Give-up flag of the single launch in host-mapped memory (host address and the address the
  // kernels store to): set by a tile whose bounded wait gave up, read and cleared by the next
  // library call on this device without any synchronisation.
  unsigned* host_flag = nullptr;
  unsigned* host_flag_dev = nullptr;
  // The current call is being captured into a HIP graph on its stream: workspaces must not
  // grow and no timing events are recorded.
  bool capturing = false;
  // the previous pipeline call: its caller stream and the done slots of its last chunk on
  // each stream (-1 if none)
  hipStream_t prev_caller = nullptr;
  int prev_done_slots[2] = {-1, -1};
  // kernel timing (pr_profile_enable)
  std::vector<hipEvent_t> ev_pool;
  struct Timed {
    hipEvent_t start, stop;
    int kind;  // 0 projection, 1 add/norm
  };
  std::vector<Timed> pending;
  double ms[2] = {0, 0};
  int launches[2] = {0, 0};
};

std::atomic<bool> g_profile{false};

std::mutex g_ctx_mu;
DevCtx* g_ctx[kMaxDevices] = {};

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

int take_event(DevCtx* c, hipEvent_t* e) {
  if (!c->ev_pool.empty()) {
    *e = c->ev_pool.back();
    c->ev_pool.pop_back();
    return PR_OK;
  }
  PR_HIP(hipEventCreate(e));
  return PR_OK;
}

// Runs launch(start, stop): with profiling on, the dispatch records its own start and end
// into two timing events (extended launch), else both are NULL.
template <typename F>
int timed(DevCtx* c, int kind, F&& launch) {
  if (!g_profile.load(std::memory_order_relaxed) || c->capturing) return launch(nullptr, nullptr);
  DevCtx::Timed t{nullptr, nullptr, kind};
  PR_TRY(take_event(c, &t.start));
  if (const int rc = take_event(c, &t.stop); rc != PR_OK) {
    c->ev_pool.push_back(t.start);
    return rc;
  }
  const int rc = launch(t.start, t.stop);
  if (rc != PR_OK) {  // nothing was recorded into the pair
    c->ev_pool.push_back(t.start);
    c->ev_pool.push_back(t.stop);
    return rc;
  }
  c->pending.push_back(t);
  return PR_OK;
}

int env_int(const char* name) {
  const char* v = std::getenv(name);
  return (v != nullptr && v[0] != '\0') ? std::atoi(v) : 0;
}

bool fault_injected() {
  const char* v = std::getenv("PR_FAULT_INJECT");
  return v != nullptr && std::strcmp(v, "launch") == 0;
}

// PR_FAULT_INJECT=wait: single-launch row reads look for an epoch no slot carries, so every
// tile's bounded wait gives up (tests of the status report).
bool wait_fault_injected() {
  const char* v = std::getenv("PR_FAULT_INJECT");
  return v != nullptr && std::strcmp(v, "wait") == 0;
}

}  // namespace

int current_device_key(std::string* key) {
  int dev = -1;
  PR_HIP(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  PR_HIP(hipGetDeviceProperties(&prop, dev));
  *key = std::string(prop.gcnArchName) + ":" + std::to_string(prop.multiProcessorCount);
  return PR_OK;
}

namespace {

int get_ctx(DevCtx** out) {
  int dev = -1;
  PR_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(PR_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lk(g_ctx_mu);
  if (g_ctx[dev] != nullptr) {
    *out = g_ctx[dev];
    return PR_OK;
  }
  hipDeviceProp_t prop;
  PR_HIP(hipGetDeviceProperties(&prop, dev));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(PR_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950", dev,
                prop.gcnArchName);
  std::unique_ptr<DevCtx> c(new DevCtx());
  c->device = dev;
  // A default-priority, non-blocking stream.  Default-flag events throughout: the dispatches
  // signal done themselves (extended launch), and a stream wait on such an event is much
  // cheaper on the host than on an event created with hipEventDisableTiming.
  hipError_t e = hipStreamCreateWithFlags(&c->sL, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreate(&c->entry);
  for (int s = 0; s < PR_NUM_SLOTS && e == hipSuccess; ++s) e = hipEventCreate(&c->done[s]);
  for (int s = 0; s < PR_NUM_SLOTS && e == hipSuccess; ++s) e = hipEventCreate(&c->ready[s]);
  c->cu_count = prop.multiProcessorCount;
  if (e == hipSuccess) {
    void* hp = nullptr;
    e = hipHostMalloc(&hp, 64, hipHostMallocMapped | hipHostMallocCoherent);
    if (e == hipSuccess) {
      c->host_flag = static_cast<unsigned*>(hp);
      __atomic_store_n(c->host_flag, 0u, __ATOMIC_RELEASE);
      e = hipHostGetDevicePointer(reinterpret_cast<void**>(&c->host_flag_dev), hp, 0);
    }
  }
  if (e != hipSuccess) {
    // release what was created; the context is not kept
    if (c->host_flag != nullptr) (void)hipHostFree(c->host_flag);
    for (int s = 0; s < PR_NUM_SLOTS; ++s) {
      if (c->done[s] != nullptr) (void)hipEventDestroy(c->done[s]);
      if (c->ready[s] != nullptr) (void)hipEventDestroy(c->ready[s]);
    }
    if (c->entry != nullptr) (void)hipEventDestroy(c->entry);
    if (c->sL != nullptr) (void)hipStreamDestroy(c->sL);
    return fail(PR_ERR_HIP, "creating the library stream and events on device %d: %s", dev,
                hipGetErrorString(e));
  }
  g_ctx[dev] = c.release();
  *out = g_ctx[dev];
  return PR_OK;
}

// The current device's context if one exists (never creates one).
int find_ctx(DevCtx** out) {
  int dev = -1;
  PR_HIP(hipGetDevice(&dev));
  *out = nullptr;
  if (dev < 0 || dev >= kMaxDevices) return fail(PR_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lk(g_ctx_mu);
  *out = g_ctx[dev];
  return PR_OK;
}

// A give-up of an earlier single launch on this device (host flag set by the kernel): reported
// once, as this call's error, and cleared.  The check reads host memory only.
int check_give_up(DevCtx* c) {
  if (c->host_flag == nullptr || __atomic_load_n(c->host_flag, __ATOMIC_ACQUIRE) == 0)
    return PR_OK;
  __atomic_store_n(c->host_flag, 0u, __ATOMIC_RELEASE);
  return fail(PR_ERR_HIP,
              "an earlier single-launch call on device %d did not complete: a tile's bounded "
              "wait for its row gave up, so that tile's output and residual rows were not "
              "written (pr_device_status reads and clears the device status bits)",
              c->device);
}

// Whether `s` is capturing into a HIP graph.  The null stream is never the capturing stream
// itself, so it is not queried.
int stream_capturing(hipStream_t s, bool* capturing) {
  *capturing = false;
  if (s == nullptr) return PR_OK;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  PR_HIP(hipStreamIsCapturing(s, &st));
  *capturing = st != hipStreamCaptureStatusNone;
  return PR_OK;
}

// Grow a device buffer.  Growing waits for all outstanding work on the device first, since
// earlier calls may still be reading the old buffer; under graph capture a buffer cannot grow
// (the call is refused before anything is enqueued).
int grow(DevCtx* c, void** p, size_t* have, size_t need) {
  if (need <= *have) return PR_OK;
  if (c->capturing)
    return fail(PR_ERR_UNSUPPORTED,
                "a workspace must grow from %zu to %zu bytes, which is not possible while the "
                "stream is capturing a graph: make one call of this shape (or a larger one) "
                "before the capture",
                *have, need);
  if (*p != nullptr) {
    PR_HIP(hipDeviceSynchronize());
    PR_HIP(hipFree(*p));
    *p = nullptr;
    *have = 0;
  }
  const hipError_t e = hipMalloc(p, need);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    *p = nullptr;
    return fail(PR_ERR_NOMEM, "workspace of %zu bytes: %s", need, hipGetErrorString(e));
  }
  *have = need;
  return PR_OK;
}

// The CU-masked stream pair reserving `cus` CUs for the add/norm.  Mask bit i enables CU i of
// the device's numbering, in which consecutive CUs lie on consecutive XCDs (checked on MI355X:
// the top n bits give n / 8 CUs on every XCD), so the top `cus` bits reserve cus / 8 CUs per
// XCD.  A CU mask belongs to a hardware queue and a process gets only a few of those, so a
// device keeps one pair: a call with another split waits for the old pair's work, destroys it
// and creates the new one (a tuning-time cost; steady-state calls reuse the pair).
int masked_pair(DevCtx* c, int cus, MaskedPair** out) {
  MaskedPair* slot = &c->masked;
  if (slot->proj != nullptr && slot->cus == cus) {
    *out = slot;
    return PR_OK;
  }
  if (c->capturing)
    return fail(PR_ERR_UNSUPPORTED, "a CU-masked stream pair cannot be created under capture");
  if (slot->proj != nullptr) {
    PR_HIP(hipStreamSynchronize(slot->proj));
    PR_HIP(hipStreamSynchronize(slot->addnorm));
    PR_HIP(hipStreamDestroy(slot->proj));
    PR_HIP(hipStreamDestroy(slot->addnorm));
    *slot = MaskedPair();
  }
  const int n = c->cu_count;
  if (cus <= 0 || cus >= n || n > 32 * 16)
    return fail(PR_ERR_UNSUPPORTED, "CU split %d on a device of %d CUs", cus, n);
  const int words = (n + 31) / 32;
  std::vector<uint32_t> mp(words, 0), ma(words, 0);
  for (int i = 0; i < n; ++i) {
    std::vector<uint32_t>& m = i < n - cus ? mp : ma;
    m[i / 32] |= 1u << (i % 32);
  }
  MaskedPair p;
  p.cus = cus;
  PR_HIP(hipExtStreamCreateWithCUMask(&p.proj, (uint32_t)words, mp.data()));
  const hipError_t e = hipExtStreamCreateWithCUMask(&p.addnorm, (uint32_t)words, ma.data());
  if (e != hipSuccess) {
    (void)hipStreamDestroy(p.proj);
    return fail(PR_ERR_HIP, "hipExtStreamCreateWithCUMask: %s", hipGetErrorString(e));
  }
  *slot = p;
  *out = slot;
  return PR_OK;
}

// Projection over M rows; launches are split by rows so that one launch's x slice stays
// below 2^30 elements (the kernel uses 32-bit offsets).
int gemm_rows(const uint16_t* x, const uint16_t* Wp, void* C, bool bf16_out, int M, int N, int K,
              const GemmCfg& cfg, long long plane_stride, hipStream_t s,
              hipEvent_t done = nullptr, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr) {
  if (fault_injected()) return fail(PR_ERR_HIP, "injected launch failure (PR_FAULT_INJECT)");
  long long rows_per = ((1LL << 30) / K) / cfg.bm * cfg.bm;
  if (rows_per <= 0) return fail(PR_ERR_SHAPE, "K=%d too large", K);
  for (long long r0 = 0; r0 < M; r0 += rows_per) {
    const int rows = (int)std::min<long long>(rows_per, M - r0);
    void* Cr = bf16_out ? (void*)(static_cast<uint16_t*>(C) + r0 * N)
                        : (void*)(static_cast<float*>(C) + r0 * N);
    const bool first = r0 == 0, last = r0 + rows_per >= M;
    // timing spans the first launch's start to the last launch's end
    PR_TRY(launch_gemm(x + r0 * K, Wp, Cr, bf16_out, rows, N, K, cfg, plane_stride, s,
                       last ? done : nullptr, t0 != nullptr && first ? t0 : nullptr,
                       t0 != nullptr && first ? (last ? t1 : nullptr) : nullptr));
    if (t0 != nullptr && last && !first) PR_HIP(hipEventRecord(t1, s));
  }
  return PR_OK;
}

int check_common(const uint16_t* x, const uint16_t* W, float* r, const float* w, float eps,
                 int T, int K, int H, int microchunk, int norm_kind, uint16_t* out) {
  return pr_validate(x, W, r, w, eps, T, K, H, microchunk, norm_kind, out);
}

uint16_t* resolve_out(DevCtx* c, uint16_t* out, int T, int H, int* rc) {
  *rc = PR_OK;
  if (out != nullptr) return out;
  *rc = grow(c, reinterpret_cast<void**>(&c->out_ws), &c->out_ws_bytes, (size_t)T * H * 2);
  if (*rc != PR_OK) return nullptr;
  c->last_borrowed = c->out_ws;
  return c->out_ws;
}

int run_conventional(DevCtx* c, const uint16_t* x, const uint16_t* W, float* r, const float* w,
                     float eps, int T, int K, int H, int norm_kind, uint16_t* out,
                     const pr_decision& d, hipStream_t s) {
  GemmCfg g;
  g.bm = d.gemm_bm;
  g.bn = d.gemm_bn;
  g.split = d.split_k;
  g.waves = d.gemm_waves;
  g.stages = d.gemm_stages;
  g.kgroups = d.gemm_kgroups;
  const long long plane = (long long)T * H;
  if (g.split == 1) {
    PR_TRY(grow(c, &c->conv, &c->conv_bytes, (size_t)plane * 2));
    PR_TRY(timed(c, 0, [&](hipEvent_t t0, hipEvent_t t1) {
      return gemm_rows(x, W, c->conv, true, T, H, K, g, plane, s, nullptr, t0, t1);
    }));
    PR_TRY(timed(c, 1, [&](hipEvent_t t0, hipEvent_t t1) {
      return launch_add_rmsnorm(c->conv, 1, 1, plane, 0, r, w, out, T, H, eps,
                                norm_kind == PR_NORM_GEMMA, 0, s, nullptr, t0, t1);
    }));
  } else {
    // K split: fp32 partial planes, summed and rounded to bf16 before the add.
    PR_TRY(grow(c, &c->conv, &c->conv_bytes, (size_t)plane * 4 * g.split));
    PR_TRY(timed(c, 0, [&](hipEvent_t t0, hipEvent_t t1) {
      return gemm_rows(x, W, c->conv, false, T, H, K, g, plane, s, nullptr, t0, t1);
    }));
    PR_TRY(timed(c, 1, [&](hipEvent_t t0, hipEvent_t t1) {
      return launch_add_rmsnorm(c->conv, 0, g.split, plane, 1, r, w, out, T, H, eps,
                                norm_kind == PR_NORM_GEMMA, 0, s, nullptr, t0, t1);
    }));
  }
  return PR_OK;
}

int run_pipeline(DevCtx* c, const uint16_t* x, const uint16_t* W, float* r, const float* w,
                 float eps, int T, int K, int H, int norm_kind, uint16_t* out,
                 const pr_decision& d, hipStream_t caller) {
  const int mc = d.microchunk;
  GemmCfg g;
  g.bm = d.gemm_bm;
  g.bn = d.gemm_bn;
  g.split = d.split_k;
  g.waves = d.gemm_waves;
  g.stages = d.gemm_stages;
  g.kgroups = d.gemm_kgroups;
  const int rows_max = std::min(mc, T);
  const long long plane = (long long)rows_max * H;  // elements of one partial plane
  const size_t slot_elems = (size_t)plane * g.split;
  if (slot_elems > c->slot_elems) {
    size_t have = c->slot_elems * PR_NUM_SLOTS * sizeof(float);
    void* p = c->slots;
    PR_TRY(grow(c, &p, &have, slot_elems * PR_NUM_SLOTS * sizeof(float)));
    c->slots = static_cast<float*>(p);
    c->slot_elems = slot_elems;
  }
  const int an_wgs = env_int("PR_FORCE_ADDNORM_WGS");
  const int delay = env_int("PR_DEBUG_DELAY");
  const bool poison = env_int("PR_DEBUG_POISON") != 0;
  const int gemma = norm_kind == PR_NORM_GEMMA;

  // The ping-pong schedule (caller stream and the library stream) or, with a CU split, the
  // partitioned one (projections and add/norms on two CU-masked library streams).
  const bool partitioned = d.addnorm_cus > 0;
  MaskedPair* mp = nullptr;
  if (partitioned) PR_TRY(masked_pair(c, d.addnorm_cus, &mp));
  std::vector<pr_plan_op> ops(8 + 8 * (size_t)d.n_chunks);
  const int n = partitioned ? pr_plan_cu_split(T, mc, ops.data(), (int)ops.size())
                            : pr_plan(T, mc, ops.data(), (int)ops.size());
  if (n < 0) return n;
  auto stream_of = [&](int id) {
    if (id == 0) return caller;
    if (partitioned) return id == 1 ? mp->proj : mp->addnorm;
    return c->sL;
  };
  int last_slot[2] = {-1, -1};  // last done slot recorded on the caller / library streams
  for (int i = 0; i < n; ++i) {
    const pr_plan_op& op = ops[i];
    float* slot = op.slot >= 0 ? c->slots + (size_t)op.slot * c->slot_elems : nullptr;
    const long long row0 = (long long)op.chunk * mc;
    hipStream_t st = stream_of(op.stream);
    // A done (ready) record that directly follows the add/norm (projection) it marks is
    // signalled by the launch.
    const bool fuse_next = op.op == PR_OP_ADDNORM && i + 1 < n &&
                           ops[i + 1].op == PR_OP_RECORD_DONE && ops[i + 1].stream == op.stream &&
                           !poison;
    const bool fuse_ready = op.op == PR_OP_GEMM && i + 1 < n &&
                            ops[i + 1].op == PR_OP_RECORD_READY &&
                            ops[i + 1].stream == op.stream && delay == 0;
    switch (op.op) {
      case PR_OP_WAIT_PREV:
        // In order on one caller stream (and joined), the previous call needs no wait; a call
        // from another stream waits for the previous call's last chunk on each stream.
        if (c->prev_caller != caller)
          for (int k = 0; k < 2; ++k)
            if (c->prev_done_slots[k] >= 0)
              PR_HIP(hipStreamWaitEvent(caller, c->done[c->prev_done_slots[k]], 0));
        break;
      case PR_OP_RECORD_ENTRY:
        PR_HIP(hipEventRecord(c->entry, caller));
        break;
      case PR_OP_WAIT_ENTRY:
        PR_HIP(hipStreamWaitEvent(st, c->entry, 0));
        break;
      case PR_OP_WAIT_DONE:
        PR_HIP(hipStreamWaitEvent(st, c->done[op.slot], 0));
        break;
      case PR_OP_GEMM:
        if (delay > 0) PR_TRY(launch_delay(delay, st));
        PR_TRY(timed(c, 0, [&](hipEvent_t t0, hipEvent_t t1) {
          return gemm_rows(x + row0 * K, W, slot, false, op.rows, H, K, g,
                           (long long)op.rows * H, st, fuse_ready ? c->ready[op.slot] : nullptr,
                           t0, t1);
        }));
        if (fuse_ready) ++i;
        break;
      case PR_OP_RECORD_READY:
        PR_HIP(hipEventRecord(c->ready[op.slot], st));
        break;
      case PR_OP_WAIT_READY:
        PR_HIP(hipStreamWaitEvent(st, c->ready[op.slot], 0));
        break;
      case PR_OP_ADDNORM:
        if (delay > 0) PR_TRY(launch_delay(delay, st));
        PR_TRY(timed(c, 1, [&](hipEvent_t t0, hipEvent_t t1) {
          return launch_add_rmsnorm(slot, 0, g.split, (long long)op.rows * H, 0, r + row0 * H,
                                    w, out + row0 * H, op.rows, H, eps, gemma, an_wgs, st,
                                    fuse_next ? c->done[op.slot] : nullptr, t0, t1);
        }));
        if (poison) PR_TRY(launch_fill_nan(slot, c->slot_elems, st));
        if (fuse_next) {
          last_slot[op.stream == 0 ? 0 : 1] = op.slot;
          ++i;
        }
        break;
      case PR_OP_RECORD_DONE:
        PR_HIP(hipEventRecord(c->done[op.slot], st));
        last_slot[op.stream == 0 ? 0 : 1] = op.slot;
        break;
      case PR_OP_JOIN:
        PR_HIP(hipStreamWaitEvent(caller, c->done[op.slot], 0));
        break;
      default:
        return fail(PR_ERR_INVALID_ARG, "bad plan op %d", op.op);
    }
  }
  c->prev_caller = caller;
  c->prev_done_slots[0] = last_slot[0];
  c->prev_done_slots[1] = last_slot[1];
  return PR_OK;
}

// Polls of a single-launch tile's wait before it gives up (each poll is a device-scope load
// and a short sleep, about a microsecond): about two seconds.  PR_SPIN_LIMIT overrides it
// (tests use small values to reach the give-up path).
unsigned spin_limit() {
  const char* v = std::getenv("PR_SPIN_LIMIT");
  if (v != nullptr && v[0] != '\0') return (unsigned)std::strtoul(v, nullptr, 10);
  return 1u << 21;
}

// The single-launch kernels over all T rows with workspace `ws` (slots and sync words set by
// the caller): one launch per block of rows whose x slice stays below 2^30 elements (32-bit
// offsets in the kernel); the launches are independent (rows do not interact) and run in
// order on `s`.  `timing`: record the library's timing events when profiling is on.
int launch_single_rows(DevCtx* c, const uint16_t* x, const uint16_t* W, float* r, const float* w,
                       float eps, int T, int K, int H, int norm_kind, uint16_t* out,
                       const GemmCfg& g, SingleWs ws, hipStream_t s, bool timing) {
  const long long rows_per = ((1LL << 30) / K) / g.bm * g.bm;
  if (rows_per <= 0) return fail(PR_ERR_SHAPE, "K=%d too large", K);
  ws.fault_mask = wait_fault_injected() ? 0x80000000u : 0u;
  ws.spin_limit = spin_limit();
  ws.host_flag = c->host_flag_dev;
  const int gemma = norm_kind == PR_NORM_GEMMA;
  for (long long r0 = 0; r0 < T; r0 += rows_per) {
    const int rows = (int)std::min<long long>(rows_per, T - r0);
    auto launch = [&](hipEvent_t t0, hipEvent_t t1) {
      return launch_gemm_add_rmsnorm(x + r0 * K, W, r + r0 * H, w, out + r0 * H, ws, rows, H, K,
                                     g, eps, gemma, s, t0, t1);
    };
    PR_TRY(timing ? timed(c, 0, launch) : launch(nullptr, nullptr));
  }
  return PR_OK;
}

GemmCfg cfg_of(const pr_decision& d) {
  GemmCfg g;
  g.bm = d.gemm_bm;
  g.bn = d.gemm_bn;
  g.split = d.split_k;
  g.waves = d.gemm_waves;
  g.stages = d.gemm_stages;
  g.kgroups = d.gemm_kgroups;
  return g;
}

// The grown single-launch workspace for T rows with configuration g (row slots, sync words,
// the pair form's words and exchange regions), as `ws` (slots, sync, pair fields).
int single_workspace(DevCtx* c, const GemmCfg& g, int T, int K, int H, SingleWs* ws) {
  // Launches cover at most 2^30 elements of x each (32-bit offsets in the kernel), in whole
  // tile rows; each launch is independent (rows do not interact).
  const long long rows_per = ((1LL << 30) / K) / g.bm * g.bm;
  if (rows_per <= 0) return fail(PR_ERR_SHAPE, "K=%d too large", K);
  const int rows_max = (int)std::min<long long>(rows_per, T);
  const bool pairs = g.split == 2;
  const size_t slots_need = (size_t)rows_max * (H / g.bn) * sizeof(unsigned long long);
  const size_t flags_need =
      pairs ? (size_t)4 * ((rows_max + 255) / 256) * (H / 256) * sizeof(unsigned long long) : 0;
  const int blocks = pairs ? 2 * ((rows_max + 255) / 256) : (rows_max + g.bm - 1) / g.bm;
  const size_t sync_need = (size_t)(3 + blocks) * sizeof(unsigned);
  // Growing any of the epoch-tagged buffers (row slots, pair words) or the sync words: the new
  // buffers are zeroed, and so are the others, since a new sync buffer restarts the device
  // epoch at 0 and a zeroed tag (epoch 0) matches no launch.  The fills run on the null stream,
  // which does not order work on a non-blocking caller stream, hence the synchronisation.
  // Steady-state calls allocate and fill nothing, so they can be captured in a graph.
  const bool grow_sync = sync_need > c->sync_bytes;
  if (slots_need > c->row_slots_bytes || flags_need > c->pair_flags_bytes || grow_sync) {
    PR_TRY(grow(c, &c->row_slots, &c->row_slots_bytes, slots_need));
    if (flags_need > 0) PR_TRY(grow(c, &c->pair_flags, &c->pair_flags_bytes, flags_need));
    if (grow_sync) {
      void* p = c->sync;
      size_t have = c->sync_bytes;
      PR_TRY(grow(c, &p, &have, sync_need));
      c->sync = static_cast<unsigned*>(p);
      c->sync_bytes = have;
      PR_HIP(hipMemset(c->sync, 0, c->sync_bytes));
    }
    PR_HIP(hipMemset(c->row_slots, 0, c->row_slots_bytes));
    if (c->pair_flags != nullptr) PR_HIP(hipMemset(c->pair_flags, 0, c->pair_flags_bytes));
    PR_HIP(hipDeviceSynchronize());
  }
  if (pairs) {
    // Exchange regions: 128 KiB per workgroup of a round and round parity; a round holds at
    // most one workgroup per CU.
    const size_t xbuf_need = (size_t)2 * kNumCUs * 128 * 1024;
    PR_TRY(grow(c, &c->xbuf, &c->xbuf_bytes, xbuf_need));
  }
  // Debug: PR_DEBUG_EPOCH=<n> stores n as the last launch's epoch before the call (tests of
  // the wrap at 2^32 - 1 launches).
  const char* dbg_epoch = std::getenv("PR_DEBUG_EPOCH");
  if (dbg_epoch != nullptr && dbg_epoch[0] != '\0') {
    if (c->capturing)
      return fail(PR_ERR_UNSUPPORTED, "PR_DEBUG_EPOCH is not supported under graph capture");
    const unsigned v = (unsigned)std::strtoul(dbg_epoch, nullptr, 10);
    PR_HIP(hipDeviceSynchronize());
    PR_HIP(hipMemcpy(c->sync + 2, &v, sizeof(v), hipMemcpyHostToDevice));
  }
  ws->slots = static_cast<unsigned long long*>(c->row_slots);
  ws->slot_words = c->row_slots_bytes / sizeof(unsigned long long);
  ws->sync = c->sync;
  ws->pwords = static_cast<unsigned long long*>(c->pair_flags);
  ws->pword_words = c->pair_flags_bytes / sizeof(unsigned long long);
  ws->xbuf = static_cast<unsigned long long*>(c->xbuf);
  ws->xbuf_words = c->xbuf_bytes / sizeof(unsigned long long);
  return PR_OK;
}

int run_single(DevCtx* c, const uint16_t* x, const uint16_t* W, float* r, const float* w,
               float eps, int T, int K, int H, int norm_kind, uint16_t* out,
               const pr_decision& d, hipStream_t s) {
  const GemmCfg g = cfg_of(d);
  if (fault_injected()) return fail(PR_ERR_HIP, "injected launch failure (PR_FAULT_INJECT)");
  SingleWs ws;
  PR_TRY(single_workspace(c, g, T, K, H, &ws));
  return launch_single_rows(c, x, W, r, w, eps, T, K, H, norm_kind, out, g, ws, s, true);
}

int run_call(const uint16_t* x, const uint16_t* W, float* r, const float* w, float eps, int T,
             int K, int H, int microchunk, int norm_kind, uint16_t* out, void* stream) {
  clear_error();
  PR_TRY(check_common(x, W, r, w, eps, T, K, H, microchunk < 0 ? 0 : microchunk, norm_kind, out));
  pr_decision d;
  PR_TRY(decide(T, K, H, microchunk, &d));
  if (log_enabled())
    std::fprintf(stderr,
                 "[proj_add_rmsnorm] T=%d K=%d H=%d path=%s mc=%d chunks=%d tile=%dx%d "
                 "split=%d reason=%d\n",
                 T, K, H,
                 d.path == PR_PATH_FUSED ? "fused"
                                         : (d.path == PR_PATH_SINGLE ? "single" : "conventional"),
                 d.microchunk,
                 d.n_chunks, d.gemm_bm, d.gemm_bn, d.split_k, d.reason);
  DevCtx* c = nullptr;
  PR_TRY(get_ctx(&c));
  PR_TRY(check_give_up(c));
  if (T == 0) return PR_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool capturing = false;
  PR_TRY(stream_capturing(s, &capturing));
  if (capturing && d.path == PR_PATH_FUSED)
    return fail(PR_ERR_UNSUPPORTED,
                "the microchunk pipeline cannot be captured in a HIP graph (it records events "
                "and waits across a library stream); under capture use the single launch or "
                "the conventional path");
  c->capturing = capturing;
  int rc = PR_OK;
  out = resolve_out(c, out, T, H, &rc);
  if (rc == PR_OK) {
    if (d.path == PR_PATH_FUSED)
      rc = run_pipeline(c, x, W, r, w, eps, T, K, H, norm_kind, out, d, s);
    else if (d.path == PR_PATH_SINGLE)
      rc = run_single(c, x, W, r, w, eps, T, K, H, norm_kind, out, d, s);
    else
      rc = run_conventional(c, x, W, r, w, eps, T, K, H, norm_kind, out, d, s);
  }
  c->capturing = false;
  return rc;
}

}  // namespace
}  // namespace pr

using namespace pr;

extern "C" {

int pr_prepare_weight(const uint16_t* W_src, int src_layout, uint16_t* W_prep, int K, int H,
                      void* stream) {
  clear_error();
  if (W_src == nullptr || W_prep == nullptr) return fail(PR_ERR_INVALID_ARG, "null weight");
  if (W_src == W_prep) return fail(PR_ERR_INVALID_ARG, "W_prep must not alias W_src");
  if (src_layout != PR_WEIGHT_OUT_IN && src_layout != PR_WEIGHT_IN_OUT)
    return fail(PR_ERR_INVALID_ARG, "unknown weight layout %d", src_layout);
  if (K <= 0 || H <= 0 || K % 64 != 0 || H % 64 != 0)
    return fail(PR_ERR_SHAPE, "K=%d and H=%d must be positive multiples of 64", K, H);
  if ((long long)K * H > (1LL << 30)) return fail(PR_ERR_SHAPE, "weight too large");
  if ((uintptr_t)W_src % 16 != 0 || (uintptr_t)W_prep % 16 != 0)
    return fail(PR_ERR_INVALID_ARG, "weights must be 16-byte aligned");
  DevCtx* c = nullptr;
  PR_TRY(get_ctx(&c));
  PR_TRY(check_give_up(c));
  return launch_prepare_weight(W_src, src_layout, W_prep, K, H, stream);
}

int pr_silu_mul(const uint16_t* gate_up, uint16_t* x, int T, int K, void* stream) {
  clear_error();
  if (T < 0 || K <= 0 || K % 64 != 0)
    return fail(PR_ERR_SHAPE, "T=%d must be >= 0 and K=%d a positive multiple of 64", T, K);
  if ((long long)T * K > (1LL << 40)) return fail(PR_ERR_SHAPE, "T=%d too large", T);
  if (T == 0) return PR_OK;
  if (gate_up == nullptr || x == nullptr) return fail(PR_ERR_INVALID_ARG, "null tensor pointer");
  if ((uintptr_t)gate_up % 16 != 0 || (uintptr_t)x % 16 != 0)
    return fail(PR_ERR_INVALID_ARG, "gate_up and x must be 16-byte aligned");
  const uintptr_t g0 = (uintptr_t)gate_up, g1 = g0 + 4ULL * T * K;
  const uintptr_t x0 = (uintptr_t)x, x1 = x0 + 2ULL * T * K;
  if (x0 < g1 && g0 < x1) return fail(PR_ERR_INVALID_ARG, "x overlaps gate_up");
  DevCtx* c = nullptr;
  PR_TRY(get_ctx(&c));
  PR_TRY(check_give_up(c));
  return launch_silu_mul(gate_up, x, T, K, stream);
}

int proj_add_rmsnorm(const uint16_t* x, const uint16_t* W, float* residual_inout,
                     const float* norm_w, float eps, int T, int K, int H, int microchunk,
                     int norm_kind, uint16_t* out, void* stream) {
  if (microchunk < 0) {
    clear_error();
    return fail(PR_ERR_MICROCHUNK, "microchunk=%d must be >= 0", microchunk);
  }
  return run_call(x, W, residual_inout, norm_w, eps, T, K, H, microchunk, norm_kind, out, stream);
}

int proj_add_rmsnorm_unfused(const uint16_t* x, const uint16_t* W, float* residual_inout,
                             const float* norm_w, float eps, int T, int K, int H, int norm_kind,
                             uint16_t* out, void* stream) {
  return run_call(x, W, residual_inout, norm_w, eps, T, K, H, -1, norm_kind, out, stream);
}

int proj_add_rmsnorm_single_launch(const uint16_t* x, const uint16_t* W, float* residual_inout,
                                   const float* norm_w, float eps, int T, int K, int H,
                                   int norm_kind, uint16_t* out, void* stream) {
  return run_call(x, W, residual_inout, norm_w, eps, T, K, H, PR_SINGLE_LAUNCH, norm_kind, out,
                  stream);
}

int pr_quantize_fp8(const uint16_t* src, uint8_t* dst, float* scales, int rows, int cols,
                    int group_rows, void* stream) {
  clear_error();
  if (rows < 0 || cols <= 0 || cols % 16 != 0)
    return fail(PR_ERR_SHAPE, "rows=%d must be >= 0 and cols=%d a positive multiple of 16", rows,
                cols);
  if (group_rows < 1) return fail(PR_ERR_INVALID_ARG, "group_rows=%d must be >= 1", group_rows);
  if ((long long)rows * cols > (1LL << 40)) return fail(PR_ERR_SHAPE, "rows=%d too large", rows);
  DevCtx* c = nullptr;
  PR_TRY(get_ctx(&c));
  PR_TRY(check_give_up(c));
  if (rows == 0) return PR_OK;
  if (src == nullptr || dst == nullptr || scales == nullptr)
    return fail(PR_ERR_INVALID_ARG, "null tensor pointer");
  if ((uintptr_t)src % 16 != 0 || (uintptr_t)dst % 16 != 0 || (uintptr_t)scales % 4 != 0)
    return fail(PR_ERR_INVALID_ARG, "src and dst must be 16-byte aligned, scales 4-byte aligned");
  const uintptr_t s0 = (uintptr_t)src, s1 = s0 + 2ULL * rows * cols;
  const uintptr_t d0 = (uintptr_t)dst, d1 = d0 + 1ULL * rows * cols;
  const uintptr_t c0 = (uintptr_t)scales, c1 = c0 + 4ULL * ((rows - 1) / group_rows + 1);
  if ((d0 < s1 && s0 < d1) || (c0 < s1 && s0 < c1) || (c0 < d1 && d0 < c1))
    return fail(PR_ERR_INVALID_ARG, "src, dst and scales must not overlap");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (quantize_fp8_single_pass(cols, group_rows))
    return launch_quantize_fp8(src, dst, scales, nullptr, rows, cols, group_rows, s);
  bool capturing = false;
  PR_TRY(stream_capturing(s, &capturing));
  c->capturing = capturing;
  int rc = grow(c, &c->row_amax, &c->row_amax_bytes, (size_t)rows * sizeof(float));
  c->capturing = false;
  if (rc != PR_OK) return rc;
  return launch_quantize_fp8(src, dst, scales, static_cast<float*>(c->row_amax), rows, cols,
                             group_rows, s);
}

int pr_prepare_weight_fp8(const uint8_t* W_src, int src_layout, uint8_t* W_prep, int K, int H,
                          void* stream) {
  clear_error();
  if (W_src == nullptr || W_prep == nullptr) return fail(PR_ERR_INVALID_ARG, "null weight");
  if (src_layout != PR_WEIGHT_OUT_IN && src_layout != PR_WEIGHT_IN_OUT)
    return fail(PR_ERR_INVALID_ARG, "unknown weight layout %d", src_layout);
  if (K <= 0 || H <= 0 || K % 64 != 0 || H % 64 != 0)
    return fail(PR_ERR_SHAPE, "K=%d and H=%d must be positive multiples of 64", K, H);
  if ((long long)K * H > (1LL << 31)) return fail(PR_ERR_SHAPE, "weight too large");
  if ((uintptr_t)W_src % 16 != 0 || (uintptr_t)W_prep % 16 != 0)
    return fail(PR_ERR_INVALID_ARG, "weights must be 16-byte aligned");
  const uintptr_t a0 = (uintptr_t)W_src, a1 = a0 + 1ULL * K * H;
  const uintptr_t b0 = (uintptr_t)W_prep, b1 = b0 + 1ULL * K * H;
  if (a0 < b1 && b0 < a1) return fail(PR_ERR_INVALID_ARG, "W_prep must not overlap W_src");
  DevCtx* c = nullptr;
  PR_TRY(get_ctx(&c));
  PR_TRY(check_give_up(c));
  return launch_prepare_weight_fp8(W_src, src_layout, W_prep, K, H, stream);
}

int proj_add_rmsnorm_fp8(const uint8_t* x_q, const float* x_scales, int scale_rows,
                         const uint8_t* W_q, const float* w_scale, float* residual_inout,
                         const float* norm_w, float eps, int T, int K, int H, int norm_kind,
                         uint16_t* out, void* stream) {
  clear_error();
  PR_TRY(pr_validate_fp8(x_q, x_scales, scale_rows, W_q, w_scale, residual_inout, norm_w, eps, T,
                         K, H, norm_kind, out));
  pr_decision d;
  PR_TRY(decide(T, K, H, PR_SINGLE_LAUNCH, &d));
  DevCtx* c = nullptr;
  PR_TRY(get_ctx(&c));
  PR_TRY(check_give_up(c));
  if (T == 0) return PR_OK;
  if (fault_injected()) return fail(PR_ERR_HIP, "injected launch failure (PR_FAULT_INJECT)");
  // The tile the time model picks, with two waves per SIMD (the FP8 loop's only forms), in two
  // K groups where the bf16 single launch uses them (one-round 256 x 128 grids) and K holds
  // whole 128-deep stages; the K-split pair form has no FP8 variant.
  GemmCfg g = cfg_of(d);
  if (g.split != 1)
    return fail(PR_ERR_UNSUPPORTED, "the K-split pair form has no FP8 variant");
  if (g.bm == 192 && g.bn == 192) {  // the bf16 launch's 12-wave tile has no FP8 form
    const GemmCfg b = choose_single(std::max(T, 1), H, K, false);
    if (b.bm == 0)
      return fail(PR_ERR_SHAPE, "single launch (FP8): H=%d is not a multiple of 128 with at "
                  "most 64 tile columns", H);
    g.bm = b.bm;
    g.bn = b.bn;
    g.kgroups = b.kgroups;
  }
  g.waves = 8;
  if (!(g.bm == 256 && g.bn == 128 && g.kgroups == 2 && K % 128 == 0)) g.kgroups = 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool capturing = false;
  PR_TRY(stream_capturing(s, &capturing));
  c->capturing = capturing;
  int rc = PR_OK;
  out = resolve_out(c, out, T, H, &rc);
  SingleWs ws;
  if (rc == PR_OK) rc = single_workspace(c, g, T, K, H, &ws);
  c->capturing = false;
  if (rc != PR_OK) return rc;
  ws.fault_mask = wait_fault_injected() ? 0x80000000u : 0u;
  ws.spin_limit = spin_limit();
  ws.host_flag = c->host_flag_dev;
  const int gemma = norm_kind == PR_NORM_GEMMA;
  const long long rows_per = ((1LL << 30) / K) / g.bm * g.bm;
  for (long long r0 = 0; r0 < T; r0 += rows_per) {
    const int rows = (int)std::min<long long>(rows_per, T - r0);
    auto launch = [&](hipEvent_t t0, hipEvent_t t1) {
      return launch_gemm_add_rmsnorm_fp8(x_q + r0 * K, W_q, residual_inout + r0 * H, norm_w,
                                         out + r0 * H, ws, rows, H, K, g, x_scales, scale_rows,
                                         (int)r0, w_scale, eps, gemma, s, t0, t1);
    };
    PR_TRY(capturing ? launch(nullptr, nullptr) : timed(c, 0, launch));
  }
  return PR_OK;
}

int pr_project_partial(const uint16_t* x, const uint16_t* W, float* y_partial, int T, int K,
                       int H, void* stream) {
  clear_error();
  if (T < 0 || K <= 0 || H <= 0 || K % 64 != 0 || H % 64 != 0)
    return fail(PR_ERR_SHAPE, "T=%d must be >= 0 and K=%d, H=%d positive multiples of 64", T, K,
                H);
  if ((long long)K * H > (1LL << 30) || (long long)T * H > (1LL << 40))
    return fail(PR_ERR_SHAPE, "sizes too large");
  DevCtx* c = nullptr;
  PR_TRY(get_ctx(&c));
  PR_TRY(check_give_up(c));
  if (T == 0) return PR_OK;
  if (x == nullptr || W == nullptr || y_partial == nullptr)
    return fail(PR_ERR_INVALID_ARG, "null tensor pointer");
  if ((uintptr_t)x % 16 != 0 || (uintptr_t)W % 16 != 0 || (uintptr_t)y_partial % 16 != 0)
    return fail(PR_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const uintptr_t y0 = (uintptr_t)y_partial, y1 = y0 + 4ULL * T * H;
  const uintptr_t x0 = (uintptr_t)x, x1 = x0 + 2ULL * T * K;
  const uintptr_t w0 = (uintptr_t)W, w1 = w0 + 2ULL * K * H;
  if ((y0 < x1 && x0 < y1) || (y0 < w1 && w0 < y1))
    return fail(PR_ERR_INVALID_ARG, "y_partial overlaps x or W");
  const GemmCfg g = choose_gemm_unsplit(T, H, K);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return timed(c, 0, [&](hipEvent_t t0, hipEvent_t t1) {
    return gemm_rows(x, W, y_partial, false, T, H, K, g, (long long)T * H, s, nullptr, t0, t1);
  });
}

int pr_add_rmsnorm_partials(const float* partials, int P, long long plane_stride,
                            float* residual_inout, const float* norm_w, float eps, int rows,
                            int H, int norm_kind, uint16_t* out, void* stream) {
  clear_error();
  if (rows < 0 || H <= 0 || H % 64 != 0)
    return fail(PR_ERR_SHAPE, "rows=%d must be >= 0 and H=%d a positive multiple of 64", rows, H);
  if (P < 1 || plane_stride < (long long)rows * H)
    return fail(PR_ERR_INVALID_ARG, "P=%d must be >= 1 and plane_stride=%lld >= rows * H", P,
                plane_stride);
  if (norm_kind != PR_NORM_STANDARD && norm_kind != PR_NORM_GEMMA)
    return fail(PR_ERR_INVALID_ARG, "unknown norm_kind %d", norm_kind);
  if (!(eps >= 0.0f) || std::isinf(eps)) return fail(PR_ERR_INVALID_ARG, "eps must be finite and >= 0");
  DevCtx* c = nullptr;
  PR_TRY(get_ctx(&c));
  PR_TRY(check_give_up(c));
  if (rows == 0) return PR_OK;
  if (partials == nullptr || residual_inout == nullptr || norm_w == nullptr || out == nullptr)
    return fail(PR_ERR_INVALID_ARG, "null tensor pointer");
  const uintptr_t a[4] = {(uintptr_t)partials, (uintptr_t)residual_inout, (uintptr_t)norm_w,
                          (uintptr_t)out};
  for (uintptr_t p : a)
    if (p % 16 != 0 || (plane_stride * 4) % 16 != 0)
      return fail(PR_ERR_INVALID_ARG, "pointers and the plane stride must be 16-byte aligned");
  struct R { uintptr_t lo, hi; };
  const R rp{(uintptr_t)partials, (uintptr_t)partials + 4ULL * ((P - 1) * plane_stride +
                                                             (long long)rows * H)};
  const R rr{(uintptr_t)residual_inout, (uintptr_t)residual_inout + 4ULL * rows * H};
  const R rn{(uintptr_t)norm_w, (uintptr_t)norm_w + 4ULL * H};
  const R ro{(uintptr_t)out, (uintptr_t)out + 2ULL * rows * H};
  auto ov = [](const R& u, const R& v) { return u.lo < v.hi && v.lo < u.hi; };
  if (ov(rr, rp) || ov(rr, rn) || ov(ro, rp) || ov(ro, rr) || ov(ro, rn))
    return fail(PR_ERR_INVALID_ARG, "the residual or out overlaps another buffer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  return timed(c, 1, [&](hipEvent_t t0, hipEvent_t t1) {
    return launch_add_rmsnorm(partials, 0, P, plane_stride, 0, residual_inout, norm_w, out, rows,
                              H, eps, norm_kind == PR_NORM_GEMMA, 0, s, nullptr, t0, t1);
  });
}

int proj_add_rmsnorm_silu(const uint16_t* gate_up, const uint16_t* W, float* residual_inout,
                          const float* norm_w, float eps, int T, int K, int H, int norm_kind,
                          uint16_t* out, void* stream) {
  clear_error();
  PR_TRY(pr_validate_silu(gate_up, W, residual_inout, norm_w, eps, T, K, H, norm_kind, out));
  pr_decision d;
  PR_TRY(decide(T, K, H, PR_SINGLE_LAUNCH, &d));
  DevCtx* c = nullptr;
  PR_TRY(get_ctx(&c));
  PR_TRY(check_give_up(c));
  if (T == 0) return PR_OK;
  if (fault_injected()) return fail(PR_ERR_HIP, "injected launch failure (PR_FAULT_INJECT)");
  // The single launch's tile, with two waves per SIMD and one K group (the forms with the
  // SiluAndMul main loop); the K-split pair form has none.
  GemmCfg g = cfg_of(d);
  if (g.split != 1)
    return fail(PR_ERR_UNSUPPORTED, "the K-split pair form has no SiluAndMul variant");
  if (g.bm == 192 && g.bn == 192) {  // the bf16 launch's 12-wave tile has no SiluAndMul form
    const GemmCfg b = choose_single(std::max(T, 1), H, K, false);
    if (b.bm == 0)
      return fail(PR_ERR_SHAPE, "single launch (SiluAndMul): H=%d is not a multiple of 128 with at "
                  "most 64 tile columns", H);
    g.bm = b.bm;
    g.bn = b.bn;
  }
  g.waves = 8;
  g.kgroups = 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool capturing = false;
  PR_TRY(stream_capturing(s, &capturing));
  c->capturing = capturing;
  int rc = PR_OK;
  out = resolve_out(c, out, T, H, &rc);
  SingleWs ws;
  if (rc == PR_OK) rc = single_workspace(c, g, T, K, H, &ws);
  c->capturing = false;
  if (rc != PR_OK) return rc;
  ws.fault_mask = wait_fault_injected() ? 0x80000000u : 0u;
  ws.spin_limit = spin_limit();
  ws.host_flag = c->host_flag_dev;
  const int gemma = norm_kind == PR_NORM_GEMMA;
  // Offsets inside a launch are 32-bit: at most 2^30 elements of gate_up per launch.
  const long long rows_per = std::max<long long>(((1LL << 30) / (2LL * K)) / g.bm * g.bm, g.bm);
  for (long long r0 = 0; r0 < T; r0 += rows_per) {
    const int rows = (int)std::min<long long>(rows_per, T - r0);
    auto launch = [&](hipEvent_t t0, hipEvent_t t1) {
      return launch_gemm_add_rmsnorm_silu(gate_up + r0 * 2 * K, W, residual_inout + r0 * H,
                                          norm_w, out + r0 * H, ws, rows, H, K, g, eps, gemma, s,
                                          t0, t1);
    };
    PR_TRY(capturing ? launch(nullptr, nullptr) : timed(c, 0, launch));
  }
  return PR_OK;
}

int pr_init(void) {
  clear_error();
  DevCtx* c = nullptr;
  PR_TRY(get_ctx(&c));
  return noalloc_setup();
}

int proj_add_rmsnorm_single_launch_noalloc(const uint16_t* x, const uint16_t* W,
                                           float* residual_inout, const float* norm_w, float eps,
                                           int T, int K, int H, int norm_kind, uint16_t* out,
                                           void* stream) {
  clear_error();
  PR_TRY(check_common(x, W, residual_inout, norm_w, eps, T, K, H, 0, norm_kind, out));
  if (T > 0 && out == nullptr)
    return fail(PR_ERR_INVALID_ARG, "out must be given: a borrowed output would be allocated");
  pr_decision d;
  PR_TRY(decide(T, K, H, PR_SINGLE_LAUNCH, &d));
  DevCtx* c = nullptr;
  PR_TRY(find_ctx(&c));
  if (c == nullptr)
    return fail(PR_ERR_UNSUPPORTED, "pr_init() has not been called on the current device");
  PR_TRY(check_give_up(c));
  if (T == 0) return PR_OK;
  if (fault_injected()) return fail(PR_ERR_HIP, "injected launch failure (PR_FAULT_INJECT)");
  const GemmCfg g = cfg_of(d);
  if (g.split != 1)
    return fail(PR_ERR_UNSUPPORTED, "the K-split pair form needs exchange regions beyond the "
                "fixed workspace");
  const char* dbg_epoch = std::getenv("PR_DEBUG_EPOCH");
  if (dbg_epoch != nullptr && dbg_epoch[0] != '\0')
    return fail(PR_ERR_UNSUPPORTED, "PR_DEBUG_EPOCH is not supported without allocation");
  SingleWs ws;
  PR_TRY(noalloc_workspace(&ws));
  // One launch covers at most rows_per rows; its slots and counters must fit the fixed array.
  const long long rows_per = std::max<long long>(((1LL << 30) / K) / g.bm * g.bm, 1);
  const long long rows_max = std::min<long long>(rows_per, T);
  const unsigned long long slots_need = (unsigned long long)rows_max * (H / g.bn);
  const unsigned long long sync_need = 3 + (rows_max + g.bm - 1) / g.bm;
  if (slots_need > kNoallocSlotWords || sync_need > kNoallocSyncWords)
    return fail(PR_ERR_SHAPE,
                "T=%d, H=%d needs %llu row slots and %llu words per launch with %dx%d tiles; "
                "the fixed workspace holds %llu and %llu",
                T, H, slots_need, sync_need, g.bm, g.bn, kNoallocSlotWords, kNoallocSyncWords);
  return launch_single_rows(c, x, W, residual_inout, norm_w, eps, T, K, H, norm_kind, out, g,
                            ws, static_cast<hipStream_t>(stream), false);
}

int pr_device_status(void* stream, unsigned* status) {
  clear_error();
  if (status == nullptr) return fail(PR_ERR_INVALID_ARG, "null status");
  *status = 0;
  DevCtx* c = nullptr;
  PR_TRY(get_ctx(&c));
  PR_HIP(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  if (c->host_flag != nullptr) __atomic_store_n(c->host_flag, 0u, __ATOMIC_RELEASE);
  // The status words of the grown workspace and of the fixed one (when set up).
  unsigned* words[2] = {c->sync, nullptr};
  SingleWs fixed;
  if (noalloc_workspace(&fixed) == PR_OK) words[1] = fixed.sync;
  clear_error();  // a fixed workspace that is not set up is not an error here
  unsigned all = 0;
  for (unsigned* wd : words) {
    if (wd == nullptr) continue;
    unsigned v = 0;
    PR_HIP(hipMemcpy(&v, wd, sizeof(v), hipMemcpyDeviceToHost));
    if (v != 0) {
      PR_HIP(hipMemset(wd, 0, sizeof(unsigned)));
      PR_HIP(hipDeviceSynchronize());
    }
    all |= v;
  }
  *status = all;
  return PR_OK;
}

int pr_release_workspace(void) {
  clear_error();
  DevCtx* c = nullptr;
  PR_TRY(get_ctx(&c));
  // Outstanding work may still read the buffers.
  PR_HIP(hipDeviceSynchronize());
  void** bufs[] = {reinterpret_cast<void**>(&c->slots), &c->conv,
                   reinterpret_cast<void**>(&c->out_ws), &c->row_slots,
                   reinterpret_cast<void**>(&c->sync), &c->pair_flags, &c->xbuf, &c->row_amax};
  for (void** b : bufs) {
    if (*b != nullptr) PR_HIP(hipFree(*b));
    *b = nullptr;
  }
  c->slot_elems = 0;
  c->conv_bytes = c->out_ws_bytes = c->row_slots_bytes = c->sync_bytes = 0;
  c->pair_flags_bytes = c->xbuf_bytes = c->row_amax_bytes = 0;
  c->last_borrowed = nullptr;
  c->prev_caller = nullptr;
  c->prev_done_slots[0] = c->prev_done_slots[1] = -1;
  return PR_OK;
}

int pr_profile_enable(int on) {
  clear_error();
  DevCtx* c = nullptr;
  PR_TRY(get_ctx(&c));
  PR_TRY(pr_profile_read(nullptr));  // drain what is pending
  c->ms[0] = c->ms[1] = 0;
  c->launches[0] = c->launches[1] = 0;
  g_profile.store(on != 0);
  return PR_OK;
}

int pr_profile_read(pr_profile* p) {
  clear_error();
  DevCtx* c = nullptr;
  PR_TRY(get_ctx(&c));
  // Every pending pair is consumed (and its events returned to the pool) even if one fails,
  // so that one bad read does not leave the queue in a state every later read fails on.
  hipError_t first_err = hipSuccess;
  for (const DevCtx::Timed& t : c->pending) {
    float ms = 0;
    hipError_t e = hipEventSynchronize(t.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.start, t.stop);
    if (e == hipSuccess) {
      c->ms[t.kind] += ms;
      c->launches[t.kind] += 1;
    } else if (first_err == hipSuccess) {
      first_err = e;
    }
    c->ev_pool.push_back(t.start);
    c->ev_pool.push_back(t.stop);
  }
  c->pending.clear();
  if (first_err != hipSuccess)
    return fail(PR_ERR_HIP, "reading kernel timing events: %s", hipGetErrorString(first_err));
  if (p != nullptr) {
    p->gemm_ms = c->ms[0];
    p->gemm_launches = c->launches[0];
    p->addnorm_ms = c->ms[1];
    p->addnorm_launches = c->launches[1];
  }
  return PR_OK;
}

const uint16_t* pr_workspace_output(void) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_ctx_mu);
  return g_ctx[dev] != nullptr ? g_ctx[dev]->last_borrowed : nullptr;
}

}  // extern "C"
