// Internal interfaces shared by the library's translation units (not part of the C ABI).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/proj_add_rmsnorm.h"

namespace pr {

// MI355X: 256 compute units (8 XCDs x 32), 2.4 GHz peak engine clock.
constexpr int kNumCUs = 256;
constexpr int kNumXCDs = 8;

// Projection tile configuration.
struct GemmCfg {
  int bm = 256;   // tile rows (tokens)
  int bn = 256;   // tile columns (hidden)
  int split = 1;  // K partitions; partial sums land in separate fp32 planes
  int waves = 4;  // waves per workgroup: 4 (one per SIMD) or 8 (two per SIMD)
  int stages = 0; // LDS ring depth; 0 = the deepest the tile fits in LDS
  int kgroups = 1; // K groups inside the workgroup (single launch, 256x128 with 8 waves: 2)
  int addnorm_cus = 0;  // pipeline: CUs reserved for the add/norm stream (0: ping-pong schedule)
};

// Tile configurations the library instantiates (rows x columns per workgroup).
constexpr int kNumTileCfgs = 3;
constexpr int kTileBM[kNumTileCfgs] = {256, 256, 128};
constexpr int kTileBN[kNumTileCfgs] = {256, 128, 128};

// Cost-model choice of tile and split for an M x N x K projection on `cus` CUs.  `fp32_out` is
// true when the projection result is kept in fp32 (the pipeline's slot), false when it is
// emitted in bf16.
GemmCfg choose_gemm(int M, int N, int K, bool fp32_out, int cus = kNumCUs);
// The same choice restricted to one K partition (a single fp32 output plane).
GemmCfg choose_gemm_unsplit(int M, int N, int K);
// Modelled time (seconds) of the projection of M x N x K with tile configuration c (index into
// kTileBM/kTileBN) and K split, including the add/norm's read of its output, when it has `cus`
// CUs and that share of the chip's power to itself (kNumCUs: alone on the GPU).
double model_gemm_time(int M, int N, int K, int c, int split, bool fp32_out, int cus);
// Tile of the single launch for an M x N x K region (bm = 0 if N fits none); with_192 = false
// keeps to the tiles that every single-launch form instantiates (FP8, SiluAndMul).
GemmCfg choose_single(int M, int N, int K, bool with_192);

// Error reporting: stores the message for pr_last_error() and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
bool log_enabled();

// Auto-mode / explicit decision (host only); `microchunk` = -1 marks the unfused entry point.
int decide(int T, int K, int H, int microchunk, pr_decision* d);

// Identity of the current device for tuning files: "<gcnArchName>:<CU count>" (runtime).
int current_device_key(std::string* key);

// Environment overrides: returns PR_OK and sets the values (0 when unset) or an error for a
// malformed value.
int read_overrides(int* mc_override, int* threshold_override);

}  // namespace pr

// ---- device-side launchers (pr_kernels.hip) -----------------------------------------------
namespace pr {

// y = x . W^T for M rows.  x [M][K] bf16 (row stride K), Wp the prepared weight (K*N).
// fp32 mode: C planes [split][M][N] at plane stride `plane_stride` elements.
// bf16 mode (split must be 1): C is [M][N] bf16, rounded to nearest even.
// done_event (a hipEvent_t or NULL) is signalled when the launch completes; start_timing /
// stop_timing (hipEvent_t or NULL) take the dispatch's own start and end times.
int launch_gemm(const uint16_t* x, const uint16_t* Wp, void* C, bool bf16_out, int M, int N,
                int K, const GemmCfg& cfg, long long plane_stride, void* stream,
                void* done_event = nullptr, void* start_timing = nullptr,
                void* stop_timing = nullptr);

// r <- r + y; out = RMSNorm(r) for `rows` rows of width H.
// y: fp32 planes [nplanes][rows][H] (summed in plane order) or bf16 [rows][H] (y_bf16 != 0).
// round_y: round the summed fp32 y to bf16 before the add (conventional semantics).
// max_wgs > 0 caps the workgroups (CUs) the launch occupies; the result does not depend on it.
int launch_add_rmsnorm(const void* y, int y_bf16, int nplanes, long long plane_stride,
                       int round_y, float* r, const float* w, uint16_t* out, int rows, int H,
                       float eps, int gemma, int max_wgs, void* stream,
                       void* done_event = nullptr, void* start_timing = nullptr,
                       void* stop_timing = nullptr);

// Device workspace of the single launch (owned by the runtime, zeroed when allocated).
//   slots: slot_words 64-bit row-partial slots, {epoch, fp32 partial}; a launch needs
//          (N / tile columns) * M of them.
//   sync:  [0] status bits (bit 0: a wait gave up after spin_limit polls), [1] finished
//          workgroups, [2] epoch of the last launch, [3 ..] one completion counter per tile
//          row (per 128-row block for the pair form); all but [0] and [2] are zero between
//          launches, and [2] advances by one per launch (on the device).
//   pwords, xbuf: the pair form's XCD-id and ready words (pword_words 64-bit words, epoch
//          tagged like the slots; 4 per 256x256 tile) and exchange regions (xbuf_words 64-bit
//          words: 16384 per workgroup of a round, twice that for launches of several rounds).
//   fault_mask: 0, or a nonzero mask that makes every wait look for an epoch no word carries
//          (tests of the give-up path); spin_limit: polls before a wait gives up.
//   host_flag: NULL, or a word of host-mapped memory that a tile whose wait gives up sets to 1
//          (the next library call on the device reads it without synchronising).
// An epoch-tagged word holding the launch's epoch was written by that launch; a cleared word
// holds epoch 0, which no launch uses.
struct SingleWs {
  unsigned long long* slots = nullptr;
  unsigned long long slot_words = 0;
  unsigned* sync = nullptr;
  unsigned long long* pwords = nullptr;
  unsigned long long pword_words = 0;
  unsigned long long* xbuf = nullptr;
  size_t xbuf_words = 0;
  unsigned fault_mask = 0;
  unsigned spin_limit = 0;
  unsigned* host_flag = nullptr;
};

// Projection, residual add and RMSNorm of M rows in one launch (tile cfg.bm x cfg.bn, 8 waves
// or the 4-wave 256x128 form; N % cfg.bn == 0, N / cfg.bn <= 64); cfg.split == 2 selects the
// pair form (256x256, 8 waves, K halves on two workgroups; N a multiple of 256, K >= 256).
int launch_gemm_add_rmsnorm(const uint16_t* x, const uint16_t* Wp, float* r, const float* w,
                            uint16_t* out, const SingleWs& ws, int M, int N, int K,
                            const GemmCfg& cfg, float eps, int gemma, void* stream,
                            void* start_timing = nullptr, void* stop_timing = nullptr);

// The single launch with the FP8 projection: xq [M][K] and the prepared Wq (E4M3 bytes,
// Wq[((k/16)*N + n)*16 + k%16] = W[n][k]); y = acc * x_scales[(scale_row0 + row) / scale_rows]
// * w_scale[0] before the residual add.  Tiles 256x256, 256x128, 128x128 with 8 waves; K a
// multiple of 64.
int launch_gemm_add_rmsnorm_fp8(const uint8_t* xq, const uint8_t* Wq, float* r, const float* w,
                                uint16_t* out, const SingleWs& ws, int M, int N, int K,
                                const GemmCfg& cfg, const float* x_scales, int scale_rows,
                                int scale_row0, const float* w_scale, float eps, int gemma,
                                void* stream, void* start_timing = nullptr,
                                void* stop_timing = nullptr);

// The single launch with SiluAndMul in the main loop: gate_up [M][2K] bf16 (gate first); the
// projection's x = bf16(silu(gate) * up) is formed per LDS stage.  Tiles 256x256, 256x128,
// 128x128 with 8 waves.
int launch_gemm_add_rmsnorm_silu(const uint16_t* gate_up, const uint16_t* Wp, float* r,
                                 const float* w, uint16_t* out, const SingleWs& ws, int M, int N,
                                 int K, const GemmCfg& cfg, float eps, int gemma, void* stream,
                                 void* start_timing = nullptr, void* stop_timing = nullptr);

int launch_prepare_weight(const uint16_t* src, int src_layout, uint16_t* dst, int K, int H,
                          void* stream);

// Fixed single-launch workspace of the entry point that allocates nothing (pr_noalloc.hip):
// kNoallocSlotWords 64-bit row-partial slots (8 MiB) and kNoallocSyncWords 32-bit words.
constexpr unsigned long long kNoallocSlotWords = 1ull << 20;
constexpr unsigned long long kNoallocSyncWords = 4096;
// Once per device, with the device current: looks up the array's device address and clears it
// (synchronises the device).
int noalloc_setup();
// The current device's fixed workspace as slots and sync words of `ws` (the other fields are
// left to the caller); PR_ERR_UNSUPPORTED when noalloc_setup has not run on the device.
int noalloc_workspace(SingleWs* ws);

// x[T][K] = bf16(silu(gate) * up) from the merged gate_up[T][2K] (gate first); K % 8 == 0,
// both 16-byte aligned.
// FP8 quantisation (pr_fp8.hip): codes [rows][cols] E4M3 of the bf16 src by groups of
// group_rows rows, scales[g] = amax / 448 (1 for an all-zero group); row_amax is a workspace of
// `rows` floats.  cols % 16 == 0.
// Groups of 1, 2 or 4 rows of at most 8192 columns are quantised in one pass, with no
// row-maximum workspace (row_amax may then be null).
bool quantize_fp8_single_pass(int cols, int group_rows);
int launch_quantize_fp8(const uint16_t* src, uint8_t* dst, float* scales, float* row_amax,
                        int rows, int cols, int group_rows, void* stream);
// FP8 weight layout: dst[((k/16)*H + h)*16 + k%16] = W[h][k] from [H][K] or [K][H] bytes.
int launch_prepare_weight_fp8(const uint8_t* src, int src_layout, uint8_t* dst, int K, int H,
                              void* stream);
int launch_silu_mul(const uint16_t* gate_up, uint16_t* x, int T, int K, void* stream);

// Debug helpers: a bounded sleep (iters x s_sleep 127) and a NaN fill.
int launch_delay(int iters, void* stream);
int launch_fill_nan(float* p, size_t n, void* stream);
// Synthetic device data for tuning: bf16 values uniform in [-scale, scale) from a counter hash.
int launch_fill_bf16_hash(uint16_t* p, size_t n, uint32_t seed, float scale, void* stream);
int launch_fill_f32_hash(float* p, size_t n, uint32_t seed, float scale, float offset,
                         void* stream);

}  // namespace pr
