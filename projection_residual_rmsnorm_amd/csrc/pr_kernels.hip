// gfx950 kernels of the projection -> residual add -> RMSNorm path.
//
//  * gemm_bf16_kernel: y = x . W^T on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16), fp32
//    accumulation, tiles staged through LDS with direct global->LDS loads, double-buffered.
//    The projection of the region ("TPSP Design" page, section 3, Fusion regions: o_proj and
//    down_proj) is the dense contraction of the path, so it is the part that runs on MFMA.
//  * add_rmsnorm_kernel: r <- r + y in fp32 (in place), then RMSNorm of the row with a
//    wavefront reduction of the sum of squares and one bf16 rounding of the output
//    ("TPSP Design" section 3: the fused path updates the residual and returns normalised
//    states; "Plugin Architecture" page, GemmaRMSNorm row: fp32 weight multiply).  HBM-bound.
//  * prepare_weight kernels: the one-time layout change of the weight after load.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <type_traits>

#include "pr_internal.h"

namespace pr {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void global_cvoid_t;

constexpr int kBK = 32;  // K depth of one LDS stage (4 groups of 8 bf16 = 64 bytes per row)
// Word 3 of a gfx9 buffer resource for raw (untyped) accesses: data format 32 bits, so the
// hardware range-checks each access against the resource's byte count.
constexpr int kBufferRsrcWord3 = 0x00020000;
// Cache-policy operand of a buffer store: sc1 (device scope).
constexpr int kStoreSc1 = 16;

// s_waitcnt encodings (gfx9): vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
// The builtin (unlike inline asm) is understood by the compiler's own wait insertion, which
// then knows which direct-to-LDS loads have landed.
#define PR_VMCNT(n) (0x0F70 | ((n)&15) | ((((n) >> 4) & 3) << 14))
#define PR_LGKMCNT0 0xC07F

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN stays a quiet NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ void load_to_lds16(const char* gbase, uint32_t lane_off,
                                              char* lds_dst_wave_base) {
  // Each lane copies 16 bytes from gbase + lane_off (gbase wave-uniform) to
  // lds_dst_wave_base + lane * 16.  The sum is formed in the global address space so that the
  // load uses the scalar-base + 32-bit vector-offset form.
  const __attribute__((address_space(1))) char* g =
      (const __attribute__((address_space(1))) char*)gbase;
  __builtin_amdgcn_global_load_lds((global_cvoid_t*)(g + lane_off),
                                   (lds_void_t*)lds_dst_wave_base, 16, 0, 0);
}

// Workgroup barrier without a memory fence (a fence would wait for every outstanding global
// load, i.e. drain the prefetch ring).  Callers wait for what they need first.
__device__ __forceinline__ void barrier_no_fence() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// --------------------------------------------------------------------------------------------
// Projection.
//
// Operands
//   A  = x [M][K] bf16, row stride K (the chunk's tokens).
//   Bp = prepared weight, Bp[((k/8)*N + n)*8 + k%8] = W[n][k].
// LDS stage layouts (bytes).  Every direct global->LDS load writes 1 KiB contiguously (lane
// l at offset 16 l), so the global side chooses which 16 bytes land where:
//   A stage: [BM rows][4 slots][16 B], row r's slot p holding k-group p ^ f(r) with
//            f(r) = (r >> 2) & 3.  One load fills 16 rows (64 B of each row, a coalesced
//            read).  The swizzle was chosen by measurement on gfx950: a 64-lane ds_read_b128
//            of a fragment (rows l % 32, k-group 2s + l / 32) takes 4.4 cycles per CU with it,
//            as a contiguous 1 KiB read does, against 8 with ((r >> 1) ^ (r >> 3)) & 3 and 16
//            with no swizzle.
//   B stage: [4 k-groups][BN columns][16 B] (lane-linear on both sides: the prepared weight
//            already has this layout).
//   With two K groups (a stage of two 32-deep halves, bf16 or FP8) the x rows are loaded as
//   whole 128-byte lines instead: one load fills 8 rows x 128 B into one [BM rows][8 slots]
//   [16 B] block for both halves, row r's slot p holding k-group p ^ ((r >> 1) & 7) of the
//   stage, and the two halves' B blocks follow it.  Measured on gfx950 with the o_proj tiles'
//   real access pattern on every CU (a load-only probe): 42 B per clock per CU against 31 for
//   two 16-row x 64-byte loads per 128-byte line; the swizzle reads a fragment in 4.25 cycles
//   per CU, as a contiguous 1 KiB read does (8 with r & 7, 24 unswizzled).
// A 32x32x16 MFMA takes, per lane l, A[row l%32][k 8*(l/32)..+8] and B[k 8*(l/32)..+8][col l%32],
// one 16-byte read each.
//
// Pipeline: NB stage buffers in a ring, stages issued NB-1 ahead.  Each stage step runs the
// MFMAs of its first k-substep while reading the second substep's fragments, waits for the
// next stage to land (own loads) and meets the other waves at one barrier, then runs the
// second substep's MFMAs while reading the next stage's first fragments.  A buffer is refilled
// one step after the barrier that follows its last read.  The loop runs whole trips of NB
// steps and then the remaining (K per split / 32) mod NB steps.
//
// Loads are latency-bound rather than bandwidth-bound: a stage is usable only once its
// slowest load (an L2 miss) has landed, so the bytes a CU keeps in flight, (NB - 1) stages,
// set its load rate.  NB is therefore as deep as the 160 KiB of LDS allows.
// --------------------------------------------------------------------------------------------

// One LDS object per ring buffer (instantiated only for the buffers a kernel uses): the
// compiler tracks direct-to-LDS loads per object, so a fragment read from one buffer does not
// wait for loads still landing in another.
template <int I, int BYTES, int BM, int BN, int NB, int WM, int WN>
__device__ __forceinline__ char* ring_buffer() {
  __shared__ __attribute__((aligned(1024))) char buf[BYTES];
  return buf;
}

// Tile order.  Workgroups are dealt round-robin to the 8 XCDs (linear id % 8); each XCD gets a
// contiguous range of the logical order, and the logical order walks groups of 8 tile rows
// column by column, so the ~32 workgroups an XCD runs at once cover an 8 x 4 patch of tiles
// and share their x rows and weight columns in that XCD's L2.
__device__ __forceinline__ int xcd_logical(int b, int total) {
  const int q8 = total / kNumXCDs;
  const int r8 = total % kNumXCDs;
  const int xcd = b % kNumXCDs;
  return xcd * q8 + (xcd < r8 ? xcd : r8) + b / kNumXCDs;
}

__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int* tm, int* tn) {
  constexpr int GROUP_M = 8;
  const int group = t / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int in_group = t % (GROUP_M * tiles_n);
  *tm = first_m + in_group % gm;
  *tn = in_group / gm;
}

template <int TM, int TN>
struct TileAcc {
  f32x16_t v[TM][TN];
};

// Main-loop tail hook: what the ring's last refills load.  With NoTail they re-read the last
// stage (the buffers are never read again); a hook with kLoads >= 0 is called instead as
// tail(j, buffer) for the j-th refill past the last stage (j = 0 .. NB-2) and must issue exactly
// kLoads direct-to-LDS loads per wave, the count of a stage, so the loop's waits stay exact.
struct NoTail {
  static constexpr int kLoads = -1;
  __device__ void operator()(int, char*) const {}
};

// Thin tail: the refills past the last stage keep the loop's load count exact with loads that
// cost next to nothing, every lane of a refill reading the same 16 bytes (one cache line for
// the whole wave) into the buffer being refilled, which is never read again.  The default
// refills re-read the last stage, a stage's worth of L2 reads per refill that the wait after
// the loop has to drain.  The main loop issues these refills itself (issue_stage_sel), with no
// branch between them and the stage refills, so that all of them can be scheduled among the
// step's MFMAs.
template <typename T, typename = void>
struct IsThin : std::false_type {};
template <typename T>
struct IsThin<T, std::void_t<decltype(T::kThin)>> : std::true_type {};

template <int LOADS>
struct ThinTail {
  static constexpr int kLoads = LOADS;
  static constexpr bool kThin = true;
};

// Main loop of one output tile: the product of A[m0 .. m0+BM)[k_begin .. k_begin + 32 KG nk)
// and the weight columns [n0 .. n0+BN) over the same K range, in the 32x32 MFMA accumulator
// layout.  Returns with each wave past its own last fragment read: callers that reuse the
// ring's LDS synchronize first.
//
// KG > 1 splits K inside the workgroup: the waves form KG groups of WM x WN waves, a stage
// holds KG consecutive 32-deep halves of K, and group g computes the whole BM x BN tile over
// half g of every stage.  Each wave then holds a partial sum over 1/KG of K (the caller adds
// the groups' partials); with KG = 2 and 4-wave groups every SIMD runs two waves while each
// wave keeps the large wave tile.
//
// FP8: A and Bp hold OCP E4M3 bytes (A [M][K] bytes, Bp[((k/16)*N + n)*16 + k%16] = W[n][k]),
// and a stage's 64 bytes per row are 64 k-values.  The stage layouts and loads are byte for
// byte those of bf16, with 16-byte k-groups of 16 values instead of 8.  One
// v_mfma_scale_f32_32x32x64_f8f6f4 (format 0 = E4M3, unit scales) per 32x32 block covers the
// stage; lane l supplies the 16-byte k-groups l/32 and 2 + l/32 of its row (A) or column (B),
// which are the two fragments the bf16 loop reads for its two 16-deep substeps.  The matrix
// core only needs A and B to take the same k order, which this gives.
//
// SILU: A points at the merged gate/up projection output [M][2K] (gate in columns [0, K), up
// in [K, 2K)) and the loop's A operand is x = bf16(silu(gate) * up) ("Plugin Architecture"
// page, SiluAndMul row).  A stage holds the gate and the up tile, loaded like the bf16 A tile;
// once a stage has landed, the workgroup converts it in place (each thread a few 16-byte
// groups: x = gate / (1 + e^-gate) * up in fp32, rounded once to bf16, the arithmetic of the
// stand-alone SiluAndMul kernel) and meets at a second barrier before any fragment read.
// 32-deep halves per LDS stage: two for the K-group tiles (one half per group) and for the
// 12-wave tile (three waves per SIMD, each running all four 16-deep substeps of a stage, so
// that its x rows load as whole lines), one otherwise.
constexpr int stage_halves(int kg, int nw) { return kg == 2 || nw == 12 ? 2 : 1; }

template <int BM, int BN, int NB, int WM, int WN, int KG = 1, typename Tail = NoTail,
          bool FP8 = false, bool SILU = false>
__device__ __forceinline__ TileAcc<BM / WM / 32, BN / WN / 32> tile_mainloop(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bp, int M, int N, int K, int m0,
    int n0, int k_begin, int nk, const Tail& tail = Tail()) {
  constexpr int GW = WM * WN;  // waves per group
  constexpr int NW = GW * KG;  // waves per workgroup (4: one per SIMD, 8: two per SIMD)
  constexpr int WTM = BM / WM;  // wave tile rows
  constexpr int WTN = BN / WN;  // wave tile columns
  constexpr int TM = WTM / 32;
  constexpr int TN = WTN / 32;
  constexpr int A_BYTES = BM * kBK * 2;
  constexpr int A_RAW = SILU ? 2 * A_BYTES : A_BYTES;  // gate and up tiles (SILU) or x
  constexpr int B_BYTES = BN * kBK * 2;
  constexpr int A_LPW = A_BYTES / 1024 / NW;  // 1 KiB loads per wave per 32-deep half
  constexpr int B_LPW = B_BYTES / 1024 / NW;
  constexpr int HS = stage_halves(KG, NW);  // 32-deep halves per stage
  constexpr int SUBS = 2 * HS / KG;         // 16-deep substeps per wave per stage
  constexpr int LPW = HS * ((SILU ? 2 : 1) * A_LPW + B_LPW);  // per stage
  constexpr int P = NB - 1;  // stages in flight ahead of the one being computed
  constexpr int CG = BN / 64;
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "load split");
  static_assert(NW % CG == 0, "B loads: waves must cover whole k-groups");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32x32");
  static_assert(NB >= 2 && NB <= 8 && NB * HS * (A_RAW + B_BYTES) <= 160 * 1024, "LDS budget");
  static_assert(LPW * (P - 1) < 64, "vmcnt range");
  static_assert(KG == 1 || KG == 2, "one or two K groups");
  static_assert(Tail::kLoads < 0 || Tail::kLoads == LPW, "a tail refill issues a stage's loads");
  static_assert(!FP8 || Tail::kLoads < 0, "FP8: no tail hook");
  static_assert(!SILU || (HS == 1 && Tail::kLoads < 0 && !FP8), "SILU: bf16, 32-deep stages");
  static_assert(!FP8 || HS == KG, "FP8: one 64-deep half per K group");

  constexpr int HALF = A_RAW + B_BYTES;  // one 32-deep half of a stage
  constexpr int STAGE = HS * HALF;
  // Whole-line x (two halves per stage): one [BM][8 slots][16 B] x block per stage, then the
  // weight block of half h at WL_B0 + h * B_BYTES.
  constexpr bool WL = HS == 2 && !SILU;
  constexpr int WL_B0 = HS * A_BYTES;
  constexpr int WL_ALPW = HS * A_LPW;  // whole-line x loads per wave per stage
  char* const sb0 = ring_buffer<0, STAGE, BM, BN, NB, WM, WN>();
  char* const sb1 = ring_buffer<1, STAGE, BM, BN, NB, WM, WN>();
  // u is a compile-time constant at every call (unrolled loops), so this folds to one object.
  auto smem = [&](int u) -> char* {
    if constexpr (NB > 2) if (u == 2) return ring_buffer<2, STAGE, BM, BN, NB, WM, WN>();
    if constexpr (NB > 3) if (u == 3) return ring_buffer<3, STAGE, BM, BN, NB, WM, WN>();
    if constexpr (NB > 4) if (u == 4) return ring_buffer<4, STAGE, BM, BN, NB, WM, WN>();
    if constexpr (NB > 5) if (u == 5) return ring_buffer<5, STAGE, BM, BN, NB, WM, WN>();
    if constexpr (NB > 6) if (u == 6) return ring_buffer<6, STAGE, BM, BN, NB, WM, WN>();
    if constexpr (NB > 7) if (u == 7) return ring_buffer<7, STAGE, BM, BN, NB, WM, WN>();
    return u == 0 ? sb0 : sb1;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int kgrp = KG == 1 ? 0 : wave / GW;  // K group
  const int wm = (KG == 1 ? wave : wave % GW) / WN;
  const int wn = wave % WN;

  // Load assignment (per half): A load i of wave w fills LDS kilobyte q = w + NW*i, rows
  // 16q .. 16q+15 (lane l: tile row 16q + l/4, slot l%4, i.e. k-group (l%4) ^ f(row)).
  // B load i of wave w fills kilobyte q = w + NW*i: k-group q / CG, 64-column group q % CG.
  // Rows and columns past the matrix edge are clamped to the last valid one: their data only
  // feeds outputs that are never stored.  Offsets are 32-bit byte offsets (the launcher keeps
  // every operand slice below 2 GiB).
  uint32_t a_off[A_LPW];
#pragma unroll
  for (int i = 0; i < A_LPW; ++i) {
    const int q = wave + NW * i;
    const int trow = q * 16 + (lane >> 2);
    const int kg = (lane & 3) ^ ((trow >> 2) & 3);
    int row = m0 + trow;
    row = row < M ? row : M - 1;
    if constexpr (FP8)
      a_off[i] = (uint32_t)(row * K + kg * 16);  // bytes: rows of K one-byte values
    else if constexpr (SILU)
      a_off[i] = (uint32_t)(row * 2 * K + kg * 8) * 2u;  // rows of 2K (gate, then up)
    else
      a_off[i] = (uint32_t)(row * K + kg * 8) * 2u;
  }
  // Whole-line x loads: load i of wave w fills LDS kilobyte q = w + NW*i, rows 8q .. 8q+7 (lane
  // l: tile row 8q + l/8, slot l%8, i.e. k-group (l%8) ^ ((row >> 1) & 7) of the stage).
  uint32_t aw_off[WL ? WL_ALPW : 1];
  if constexpr (WL) {
#pragma unroll
    for (int i = 0; i < WL_ALPW; ++i) {
      const int q = wave + NW * i;
      const int trow = q * 8 + (lane >> 3);
      const int kg = (lane & 7) ^ ((trow >> 1) & 7);
      int row = m0 + trow;
      row = row < M ? row : M - 1;
      aw_off[i] = FP8 ? (uint32_t)(row * K + kg * 16) : (uint32_t)(row * K + kg * 8) * 2u;
    }
  }
  int b_col = n0 + (wave % CG) * 64 + lane;
  b_col = b_col < N ? b_col : N - 1;
  const uint32_t b_lane_off = (uint32_t)(((wave / CG) * N + b_col) * 8) * 2u;
  const uint32_t b_step = (uint32_t)((NW / CG) * N * 8) * 2u;

  // Stage bases advance by a fixed number of bytes per half (scalar arithmetic only).
  const char* a_base0 = FP8 ? reinterpret_cast<const char*>(A) + k_begin
                            : reinterpret_cast<const char*>(A + k_begin);
  const char* b_base0 =
      FP8 ? reinterpret_cast<const char*>(Bp) + (long long)(k_begin / 16) * N * 16
          : reinterpret_cast<const char*>(Bp + (long long)(k_begin / 8) * N * 8);
  const long long b_half_bytes = (long long)(kBK / 8) * N * 16;
  // With a thin tail: a stage's loads, or (thin) its thin refill, with no branch around the
  // loads, so that they can be scheduled between the step's MFMAs.  A thin refill reads the
  // first 16 bytes of stage 0 with every lane (the stage offset zeroed, the lane offsets
  // masked) into the buffer being refilled, which is never read again.
  auto issue_stage_sel = [&](int kt, char* buf, bool thin) {
    const uint32_t keep = thin ? 0u : 0xFFFFFFFFu;  // wave-uniform
    const long long ks = thin ? 0 : (long long)kt;
    if constexpr (WL) {
      const char* a_base = a_base0 + ks * (HS * kBK * 2);
#pragma unroll
      for (int i = 0; i < WL_ALPW; ++i)
        load_to_lds16(a_base, aw_off[i] & keep, buf + (wave + NW * i) * 1024);
#pragma unroll
      for (int h = 0; h < HS; ++h) {
        const char* b_base = b_base0 + (ks * HS + (thin ? 0 : h)) * b_half_bytes;
#pragma unroll
        for (int i = 0; i < B_LPW; ++i)
          load_to_lds16(b_base, (b_lane_off + i * b_step) & keep,
                        buf + WL_B0 + h * B_BYTES + (wave + NW * i) * 1024);
      }
      return;
    }
#pragma unroll
    for (int h = 0; h < HS; ++h) {
      const long long hs = ks * HS + (thin ? 0 : h);
      const char* a_base = a_base0 + hs * (kBK * 2);
      const char* b_base = b_base0 + hs * b_half_bytes;
      char* hb = buf + h * HALF;
#pragma unroll
      for (int i = 0; i < A_LPW; ++i)
        load_to_lds16(a_base, a_off[i] & keep, hb + (wave + NW * i) * 1024);
#pragma unroll
      for (int i = 0; i < B_LPW; ++i)
        load_to_lds16(b_base, (b_lane_off + i * b_step) & keep,
                      hb + A_RAW + (wave + NW * i) * 1024);
    }
  };
  auto issue_stage = [&](int kt, char* buf) {
    if constexpr (WL) {
      const char* a_base = a_base0 + (long long)kt * (HS * kBK * 2);
#pragma unroll
      for (int i = 0; i < WL_ALPW; ++i)
        load_to_lds16(a_base, aw_off[i], buf + (wave + NW * i) * 1024);
#pragma unroll
      for (int h = 0; h < HS; ++h) {
        const char* b_base = b_base0 + (kt * HS + h) * b_half_bytes;
#pragma unroll
        for (int i = 0; i < B_LPW; ++i)
          load_to_lds16(b_base, b_lane_off + i * b_step,
                        buf + WL_B0 + h * B_BYTES + (wave + NW * i) * 1024);
      }
      return;
    }
#pragma unroll
    for (int h = 0; h < HS; ++h) {
      const char* a_base = a_base0 + (kt * HS + h) * (kBK * 2);
      const char* b_base = b_base0 + (kt * HS + h) * b_half_bytes;
      char* hb = buf + h * HALF;
#pragma unroll
      for (int i = 0; i < A_LPW; ++i) load_to_lds16(a_base, a_off[i], hb + (wave + NW * i) * 1024);
      if constexpr (SILU) {
        // the up tile: the same rows, K columns further
#pragma unroll
        for (int i = 0; i < A_LPW; ++i)
          load_to_lds16(a_base + (long long)K * 2, a_off[i],
                        hb + A_BYTES + (wave + NW * i) * 1024);
      }
#pragma unroll
      for (int i = 0; i < B_LPW; ++i)
        load_to_lds16(b_base, b_lane_off + i * b_step, hb + A_RAW + (wave + NW * i) * 1024);
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // A fragment read: lane l reads tile row 32 rb + l%32, k-group 2s + l/32, i.e. slot
  // (2s + l/32) ^ f(row); f(row) depends only on l%32 (32 rb is a multiple of 16).
  const int a_r = lane & 31;
  const int a_f = (a_r >> 2) & 3;
  const int a_lane0 = a_r * 64 + (((lane >> 5)) ^ a_f) * 16;      // substep 0
  const int a_lane1 = a_r * 64 + ((2 + (lane >> 5)) ^ a_f) * 16;  // substep 1
  // Whole-line x: half h of a stage is slots 4h .. 4h+3 of its 128-byte rows.  With two K
  // groups group g reads half g (substeps 0, 1); with one group a wave reads both halves
  // (substeps 0 .. 3, substep s in half s / 2), and half 1's slot differs from half 0's in bit
  // 2, which the swizzle leaves an XOR of 64 bytes.
  const int w_f = (a_r >> 1) & 7;
  const int aw_lane0 = a_r * 128 + ((4 * kgrp + (lane >> 5)) ^ w_f) * 16;      // substep 0
  const int aw_lane1 = a_r * 128 + ((4 * kgrp + 2 + (lane >> 5)) ^ w_f) * 16;  // substep 1
  auto load_frags = [&](const char* stage, int s, bf16x8_t* af, bf16x8_t* bfr) {
    if constexpr (WL) {
      const int hs = s >> 1, sh = s & 1;  // (compile-time) half and substep within it
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int rb = wm * TM + i;
        af[i] = *reinterpret_cast<const bf16x8_t*>(stage + rb * 4096 +
                                                   ((sh == 0 ? aw_lane0 : aw_lane1) ^ (hs * 64)));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = wn * WTN + j * 32;
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(
            stage + WL_B0 + (kgrp + hs) * B_BYTES +
            ((2 * sh + (lane >> 5)) * BN + col + (lane & 31)) * 16);
      }
      return;
    }
    const char* buf = KG == 1 ? stage : stage + kgrp * HALF;  // this group's half
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int rb = wm * TM + i;
      af[i] = *reinterpret_cast<const bf16x8_t*>(buf + rb * 2048 + (s == 0 ? a_lane0 : a_lane1));
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = wn * WTN + j * 32;
      bfr[j] = *reinterpret_cast<const bf16x8_t*>(
          buf + A_RAW + ((2 * s + (lane >> 5)) * BN + col + (lane & 31)) * 16);
    }
  };
  // Blocks in snake order: each MFMA shares an operand with the one before it, so fewer
  // matrix-core inputs toggle (the clock under MFMA load is power-limited).  Every accumulator
  // still takes its k-steps in the same order, so results are unchanged.
  auto mfmas = [&](const bf16x8_t* af, const bf16x8_t* bfr) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jj = 0; jj < TN; ++jj) {
        const int j = (i & 1) ? TN - 1 - jj : jj;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
  };
  // One LDS fragment read after each MFMA while both last (wave tiles with fewer MFMAs than
  // fragments, such as 3 x 1 blocks, end with reads), then the rest.
  auto interleave = [&]() {
    constexpr int NMF = TM * TN, NRD = TM + TN;
#pragma unroll
    for (int g = 0; g < (NMF < NRD ? NMF : NRD); ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (NMF >= NRD) __builtin_amdgcn_sched_group_barrier(0x008, NMF - NRD, 0);
    else __builtin_amdgcn_sched_group_barrier(0x100, NRD - NMF, 0);
  };
  // The same with the step's refill loads placed one after each of the first MFMAs (used with
  // a thin tail: 3% faster on o_proj's two-K-group tile in ten alternating rounds, neutral to
  // slightly slower on the 256 x 256 tiles, which keep all loads ahead of the MFMAs).
  auto interleave_v = [&]() {
#pragma unroll
    for (int g = 0; g < TM * TN; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (g < TM + TN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (g < LPW) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    }
  };

  bf16x8_t fa0[TM], fb0[TN], fa1[TM], fb1[TN];

  if constexpr (FP8) {
    // A stage's fragments: per B column block and A row block, k-groups l/32 and 2 + l/32 of
    // the lane's row or column, joined into the 32-byte operand.  The group's 64-deep half: its
    // B block, and its x slots (whole-line) or x block.
    i32x8_t f8a[TM], f8b[TN];
    auto load_a8 = [&](const char* stage, int i) {
      const char* buf = KG == 1 ? stage : stage + kgrp * HALF;
      const char* rowp = WL ? stage + (wm * TM + i) * 4096 : buf + (wm * TM + i) * 2048;
      const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(rowp + (WL ? aw_lane0 : a_lane0));
      const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(rowp + (WL ? aw_lane1 : a_lane1));
      f8a[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto load_b8 = [&](const char* stage, int j) {
      const char* buf = KG == 1 ? stage : stage + kgrp * HALF;
      const char* bblk = WL ? stage + WL_B0 + kgrp * B_BYTES : buf + A_RAW;
      const int col = wn * WTN + j * 32 + (lane & 31);
      const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(bblk + ((lane >> 5) * BN + col) * 16);
      const i32x4_t hi =
          *reinterpret_cast<const i32x4_t*>(bblk + ((2 + (lane >> 5)) * BN + col) * 16);
      f8b[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto mf8 = [&](int i, int j) {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f8a[i], f8b[j], acc[i][j], 0,
                                                                  0, 0, 127, 0, 127);
    };
    // Prologue: stages 0 .. P-1 in flight, wait for stage 0, read its fragments.
#pragma unroll
    for (int p = 0; p < P; ++p) issue_stage(min(p, nk - 1), smem(p));
    __builtin_amdgcn_s_waitcnt(PR_VMCNT(LPW * (P - 1)));
    barrier_no_fence();
#pragma unroll
    for (int j = 0; j < TN; ++j) load_b8(smem(0), j);
#pragma unroll
    for (int i = 0; i < TM; ++i) load_a8(smem(0), i);
    // A step: the refill and the MFMAs of the stage's first half of row blocks; then (stage
    // kt+1 landed, every wave past the barrier) the next stage's first-half A fragments are
    // read while the second half's MFMAs run, and its B and second-half A fragments after them
    // (on down_proj's 256 x 256 tile 208.3 -> 200.3 us against reading all of them after the
    // barrier, outputs bitwise equal).
    constexpr int TH = (TM + 1) / 2;
    auto step8 = [&](int kt, char* next, char* refill) {
      issue_stage(min(kt + P, nk - 1), refill);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TH; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mf8(i, j);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(PR_VMCNT(LPW * (P - 1)));  // stage kt+1 landed
      __builtin_amdgcn_s_waitcnt(PR_LGKMCNT0);
      barrier_no_fence();
#pragma unroll
      for (int i = 0; i < TH; ++i) load_a8(next, i);
#pragma unroll
      for (int i = TH; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mf8(i, j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < TN; ++j) load_b8(next, j);
#pragma unroll
      for (int i = TH; i < TM; ++i) load_a8(next, i);
      __builtin_amdgcn_sched_barrier(0);
    };
    int kt = 0;
    for (; kt + NB <= nk; kt += NB) {
#pragma unroll
      for (int u = 0; u < NB; ++u) step8(kt + u, smem((u + 1) % NB), smem((u + P) % NB));
    }
    const int rem = nk - kt;
#pragma unroll
    for (int u = 0; u < NB - 1; ++u)
      if (u < rem) step8(kt + u, smem((u + 1) % NB), smem((u + P) % NB));
    TileAcc<TM, TN> res;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) res.v[i][j] = acc[i][j];
    return res;
  }

  if constexpr (SILU) {
    // In-place SiluAndMul of a landed stage: 16-byte group q of the gate tile and the same
    // group of the up tile (same row and k-group, same swizzled position) give group q of x.
    constexpr int NT = NW * 64;
    constexpr int GROUPS = A_BYTES / 16;
    static_assert(GROUPS % NT == 0, "whole groups per thread");
    auto convert = [&](char* buf) {
#pragma unroll
      for (int q0 = 0; q0 < GROUPS; q0 += NT) {
        const int q = q0 + (int)threadIdx.x;
        const u32x4_t gv = *reinterpret_cast<const u32x4_t*>(buf + q * 16);
        const u32x4_t uv = *reinterpret_cast<const u32x4_t*>(buf + A_BYTES + q * 16);
        u32x4_t xv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float g0 = bf16_to_f32(gv[j] & 0xffffu), g1 = bf16_to_f32(gv[j] >> 16);
          const float u0 = bf16_to_f32(uv[j] & 0xffffu), u1 = bf16_to_f32(uv[j] >> 16);
          const float x0 = g0 / (1.0f + __expf(-g0)) * u0;
          const float x1 = g1 / (1.0f + __expf(-g1)) * u1;
          xv[j] = f32_to_bf16_rne(x0) | (f32_to_bf16_rne(x1) << 16);
        }
        *reinterpret_cast<u32x4_t*>(buf + q * 16) = xv;
      }
    };
    // Prologue: stages 0 .. P-1 in flight, wait for stage 0, convert it, read its first
    // fragments.
#pragma unroll
    for (int p = 0; p < P; ++p) issue_stage(min(p, nk - 1), smem(p));
    __builtin_amdgcn_s_waitcnt(PR_VMCNT(LPW * (P - 1)));
    barrier_no_fence();
    convert(smem(0));
    __builtin_amdgcn_s_waitcnt(PR_LGKMCNT0);
    barrier_no_fence();
    load_frags(smem(0), 0, fa0, fb0);
    // A step: the refill; the stage's first substep; (stage kt+1's gate and up landed for
    // every wave) the second substep's MFMAs while stage kt+1 is converted; (every wave's
    // conversion written) the next stage's first fragments.
    auto step_silu = [&](int kt, char* cur, char* next, char* refill) {
      issue_stage(min(kt + P, nk - 1), refill);
      __builtin_amdgcn_sched_barrier(0);
      load_frags(cur, 1, fa1, fb1);
      mfmas(fa0, fb0);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(PR_VMCNT(LPW * (P - 1)));  // stage kt+1 landed
      __builtin_amdgcn_s_waitcnt(PR_LGKMCNT0);
      barrier_no_fence();
      mfmas(fa1, fb1);
      convert(next);
      __builtin_amdgcn_s_waitcnt(PR_LGKMCNT0);
      barrier_no_fence();
      load_frags(next, 0, fa0, fb0);
      __builtin_amdgcn_sched_barrier(0);
    };
    int kt = 0;
    for (; kt + NB <= nk; kt += NB) {
#pragma unroll
      for (int u = 0; u < NB; ++u)
        step_silu(kt + u, smem(u), smem((u + 1) % NB), smem((u + P) % NB));
    }
    const int rem = nk - kt;
#pragma unroll
    for (int u = 0; u < NB - 1; ++u)
      if (u < rem) step_silu(kt + u, smem(u), smem((u + 1) % NB), smem((u + P) % NB));
    TileAcc<TM, TN> res;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) res.v[i][j] = acc[i][j];
    return res;
  }

  // Prologue: stages 0 .. P-1 in flight, wait for stage 0, read its first fragments.
#pragma unroll
  for (int p = 0; p < P; ++p) issue_stage(min(p, nk - 1), smem(p));
  __builtin_amdgcn_s_waitcnt(PR_VMCNT(LPW * (P - 1)));
  barrier_no_fence();
  load_frags(smem(0), 0, fa0, fb0);

  // The refill is issued in every step so that the count of loads in flight is the same in
  // every step; past the last stage it re-reads the last stage (an L2 hit) into the buffer
  // being refilled, which is never read again, or runs the tail hook.
  auto step = [&](int kt, char* cur, char* next, char* refill) {
    if constexpr (SUBS == 4) {
      // 12-wave tile: four substeps per stage, fragments double-buffered across them.
      issue_stage(min(kt + P, nk - 1), refill);
      __builtin_amdgcn_sched_barrier(0);
      load_frags(cur, 1, fa1, fb1);
      mfmas(fa0, fb0);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      load_frags(cur, 2, fa0, fb0);
      mfmas(fa1, fb1);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      load_frags(cur, 3, fa1, fb1);
      mfmas(fa0, fb0);
      interleave();
    } else if constexpr (IsThin<Tail>::value) {
      const bool thin = kt + P >= nk;
      issue_stage_sel(thin ? 0 : kt + P, refill, thin);
      load_frags(cur, 1, fa1, fb1);
      mfmas(fa0, fb0);
      interleave_v();
    } else {
      if constexpr (Tail::kLoads >= 0) {
        if (kt + P >= nk)
          tail(kt + P - nk, refill);
        else
          issue_stage(kt + P, refill);
      } else {
        issue_stage(min(kt + P, nk - 1), refill);
      }
      __builtin_amdgcn_sched_barrier(0);
      load_frags(cur, 1, fa1, fb1);
      mfmas(fa0, fb0);
      interleave();
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(PR_VMCNT(LPW * (P - 1)));  // stage kt+1 landed
    __builtin_amdgcn_s_waitcnt(PR_LGKMCNT0);
    barrier_no_fence();
    load_frags(next, 0, fa0, fb0);
    mfmas(fa1, fb1);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
  };

  int kt = 0;
  for (; kt + NB <= nk; kt += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u)
      step(kt + u, smem(u), smem((u + 1) % NB), smem((u + P) % NB));
  }
  // Remaining steps: the ring position continues at buffer 0 (kt is a multiple of NB).
  const int rem = nk - kt;
#pragma unroll
  for (int u = 0; u < NB - 1; ++u)
    if (u < rem) step(kt + u, smem(u), smem((u + 1) % NB), smem((u + P) % NB));
  TileAcc<TM, TN> res;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) res.v[i][j] = acc[i][j];
  return res;
}

template <int BM, int BN, int NB, int WM, int WN>
__global__ void __launch_bounds__(WM* WN * 64, 1)
    gemm_bf16_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bp,
                     float* __restrict__ Cf, uint16_t* __restrict__ Cb, int M, int N, int K,
                     int k_split_len, long long plane_stride, int tiles_m, int tiles_n,
                     int split) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM;
  constexpr int WTN = BN / WN;
  constexpr int TM = WTM / 32;
  constexpr int TN = WTN / 32;
  constexpr int STAGE = (BM + BN) * kBK * 2;
  char* const sb0 = ring_buffer<0, STAGE, BM, BN, NB, WM, WN>();
  char* const sb1 = ring_buffer<1, STAGE, BM, BN, NB, WM, WN>();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;

  const int total = tiles_m * tiles_n * split;
  const int logical = xcd_logical(blockIdx.x, total);
  const int per_split = tiles_m * tiles_n;
  const int z = logical / per_split;
  int tm, tn;
  tile_coords(logical % per_split, tiles_m, tiles_n, &tm, &tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const TileAcc<TM, TN> tacc = tile_mainloop<BM, BN, NB, WM, WN>(
      A, Bp, M, N, K, m0, n0, z * k_split_len, k_split_len / kBK);
  const auto& acc = tacc.v;

  // Epilogue.  32x32 fp32 accumulator layout: lane l, element e holds
  // row 8*(e/4) + 4*(l/32) + e%4, column l%32.  Each wave passes its tile through its own LDS
  // region 16 rows at a time (row stride padded by 4 floats) and writes it back with 16-byte,
  // row-contiguous stores.  The regions live in the first two stage buffers.
  __syncthreads();  // every wave is past its last fragment read of the stage buffers
  constexpr int EP_LD = WTN + 4;            // floats per staged row
  constexpr int EP_BYTES = 16 * EP_LD * 4;  // one 16-row slice of a wave tile
  constexpr int EP_PER_BUF = STAGE / EP_BYTES;
  static_assert(NW <= 2 * EP_PER_BUF, "epilogue staging must fit in two stage buffers");
  float* ep = reinterpret_cast<float*>((wave < EP_PER_BUF ? sb0 : sb1) +
                                       (wave % EP_PER_BUF) * EP_BYTES);
  constexpr int LPR = WTN / 4;  // lanes per staged row (4 floats each)
  constexpr int RPI = 64 / LPR; // rows per read instruction
  const int rcol = (lane % LPR) * 4;
  const int col = n0 + wn * WTN + rcol;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 8 * h; e < 8 * h + 8; ++e)
          ep[(((e >> 2) - 2 * h) * 8 + (lane >> 5) * 4 + (e & 3)) * EP_LD + j * 32 + (lane & 31)] =
              acc[i][j][e];
      __builtin_amdgcn_s_waitcnt(PR_LGKMCNT0);
#pragma unroll
      for (int rr = 0; rr < 16 / RPI; ++rr) {
        const int r_in = rr * RPI + lane / LPR;
        const float4 v = *reinterpret_cast<const float4*>(ep + r_in * EP_LD + rcol);
        const int row = m0 + wm * WTM + i * 32 + h * 16 + r_in;
        if (row < M && col < N) {
          if (Cf != nullptr) {
            *reinterpret_cast<float4*>(Cf + (long long)z * plane_stride + (long long)row * N +
                                       col) = v;
          } else {
            const uint32_t lo = f32_to_bf16_rne(v.x) | (f32_to_bf16_rne(v.y) << 16);
            const uint32_t hi = f32_to_bf16_rne(v.z) | (f32_to_bf16_rne(v.w) << 16);
            *reinterpret_cast<uint2*>(Cb + (long long)row * N + col) = make_uint2(lo, hi);
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(PR_LGKMCNT0);  // reads done before the next slice overwrites
    }
  }
}

// --------------------------------------------------------------------------------------------
// Single-launch projection + residual add + RMSNorm.
//
// The microchunk pipeline's hand-offs ("TPSP Design" page, section 3: chunk results pass
// through reusable slots guarded by readiness and completion events) become in-kernel ones:
// the chunk is one tile row (BM tokens), the slot is the tile's own accumulators, and the
// events are device-memory words.  Each workgroup
//   1. loads its tile's residual into registers (tiles where it fits: 64 registers per lane
//      with two waves per SIMD, 128 with one) and runs the projection main loop of its BM x BN
//      tile,
//   2. forms r + y in fp32 (the fused mode's unrounded y), keeps it in registers and takes,
//      per token, the sum of squares over its BN columns (lane partials in column order,
//      reduced over the lanes of a row, then over the waves of the tile in wave order),
//   3. publishes each token's partial in a 64-bit slot {call epoch, value} and adds one to its
//      tile row's counter,
//   4. waits (one lane, bounded) until the counter shows every tile of the row, reads the
//      row's slots in tile-column order (re-reading any slot that does not yet carry this
//      call's epoch, read_epoch, bounded) and forms 1/sqrt(sum/H + eps),
//   5. writes the updated residual and the bf16 output of its tile (both after the wait, so a
//      tile whose wait gives up writes neither).
// Slots and counters are written and read with device-scope atomic stores, loads and adds, so
// no cache-wide fence is needed: a slot's epoch says whether its value is this call's.  r + y
// stays in registers from step 2 to step 5, so HBM traffic beyond the projection is the
// method's minimum: read r, write r, write out.
//
// Rounds: round q covers tile rows [q R, q R + R) with R * tiles_n workgroups, and the grid is
// never larger than the workgroups the GPU holds at once.  A wait only involves tiles of the
// same round, and a tile reaches step 3 without waiting on anything, so the waits end once
// the launch's workgroups have been placed (which needs only CU slots that other kernels
// free by finishing).  A wait that exceeds spin_limit polls gives up (status bit 0 is set, the
// host flag too, and the tile writes neither residual nor output), so every workgroup exits in
// any case.  read_epoch equals epoch;
// a test of the give-up path passes one that no slot carries.
// sync: [0] status bits, [1] workgroups finished, [2 ..] per tile row counters.  All are zero
// before the launch; the last workgroup to finish sets [1 ..] back to zero.
// slots: tiles_n columns of M 64-bit slots (slot of row t and tile column q at q * M + t, so
// the slot accesses of a wave are contiguous).
// --------------------------------------------------------------------------------------------
// Launch epochs.  sync[2] holds the epoch of the last launch; a launch uses one more.  Every
// workgroup reads it at its start, and only the launch's last workgroup to finish (when every
// other workgroup has finished) advances it, so all workgroups of a launch agree without any
// host involvement and a captured launch replays with a fresh epoch each time.  A cleared word
// carries epoch 0, which no launch uses.  Wave-uniform.
__device__ __forceinline__ unsigned launch_epoch(const unsigned* sync) {
  return __builtin_amdgcn_readfirstlane(
             __hip_atomic_load(sync + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) + 1u;
}

// End of a launch, run by all threads of its last workgroup: the `ncounters` completion
// counters (sync[3 ..]) and the finished count back to zero, and the epoch advanced.  The
// launch that used the last 32-bit epoch first clears every epoch-tagged word (both buffers,
// n0 and n1 words) so that the restarted epochs cannot meet a stale tag.
__device__ void finish_launch(unsigned* sync, int ncounters, unsigned epoch,
                              unsigned long long* tagged0, unsigned long long n0,
                              unsigned long long* tagged1, unsigned long long n1) {
  for (int i = threadIdx.x; i < ncounters; i += blockDim.x)
    __hip_atomic_store(sync + 3 + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool wrap = epoch == 0xFFFFFFFFu;
  if (wrap) {
    for (unsigned long long i = threadIdx.x; i < n0; i += blockDim.x)
      __hip_atomic_store(tagged0 + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (unsigned long long i = threadIdx.x; i < n1; i += blockDim.x)
      __hip_atomic_store(tagged1 + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_store(sync + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(sync + 2, wrap ? 0u : epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// A tile's wait gave up: status bit 0 in the device word sync[0] (read by pr_device_status)
// and, when the runtime provides one, a flag in host-mapped memory that the next library call
// on the device reads without synchronising (a system-scope vector store; many tiles may
// store the same 1).
__device__ __forceinline__ void report_give_up(unsigned* sync, unsigned* host_flag) {
  __hip_atomic_fetch_or(sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (host_flag != nullptr)
    __hip_atomic_store(host_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Sum over each group of LANES consecutive lanes (8 or 16, within one 16-lane DPP row); every
// lane of the group gets the same value (each step adds a lane and its partner, which is
// commutative, so the partners' results are bitwise equal).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int LANES>
__device__ __forceinline__ float lane_group_sum(float q) {
  static_assert(LANES == 8 || LANES == 16, "DPP row reduction over 8 or 16 lanes");
  q += dpp_mov<0xB1>(q);   // quad_perm [1,0,3,2]: partner lane ^ 1
  q += dpp_mov<0x4E>(q);   // quad_perm [2,3,0,1]: partner lane ^ 2
  q += dpp_mov<0x141>(q);  // row_half_mirror: the other quad of the 8
  if constexpr (LANES == 16) q += dpp_mov<0x140>(q);  // row_mirror: the other half-row
  return q;
}

#ifdef PR_PHASE_STAMPS
// Phase stamps, compiled only into the diagnostic library libprojaddnorm_stamps.so (the
// default library contains none of this).  Thread 0 of each of the first kStampGroups
// workgroups of a single launch records, in its first round:
//   [0]      its XCC id,
//   [1 + p]  the constant 100 MHz clock (s_memrealtime) at phase boundary p of
//            gemm_add_rmsnorm_kernel: 0 tile start, 1 main loop done, 2 K groups combined,
//            3 r + y and row sums staged, 4 row partials published, 5 row counter complete,
//            6 row slots read, 7 the wave's residual and output stores acknowledged,
//   [10], [11] the shader clock (s_memtime) at boundaries 0 and 1, so that their difference
//            over that of [1] and [2] is the clock the main loop ran at.
// Every launch overwrites the same words.
constexpr int kStampGroups = 4096;
constexpr int kStampWords = 12;
__device__ unsigned long long pr_phase_stamps[kStampGroups * kStampWords];

__device__ __forceinline__ void phase_stamp(int round, int p) {
  if (threadIdx.x != 0 || round != 0 || blockIdx.x >= kStampGroups) return;
  unsigned long long* s = pr_phase_stamps + blockIdx.x * kStampWords;
  if (p == 7) __builtin_amdgcn_s_waitcnt(0);  // this wave's stores acknowledged
  s[1 + p] = __builtin_amdgcn_s_memrealtime();
  if (p <= 1) s[10 + p] = __builtin_amdgcn_s_memtime();
  if (p == 0) {
    unsigned xcc = 0;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    s[0] = xcc & 0xff;
  }
}
#define PR_PHASE(p) phase_stamp(round, p)
#else
#define PR_PHASE(p) ((void)0)
#endif

// FP8: A and Bp point at E4M3 bytes (see tile_mainloop) and y = acc * x_scales[(scale_row0 +
// row) / scale_rows] * w_scale[0] in fp32 before the residual add; otherwise those arguments
// are unused.
// SILU: A is the merged gate/up output [M][2K] and the projection's x is SiluAndMul of it,
// formed in the main loop (see tile_mainloop).
template <int BM, int BN, int NB, int WM, int WN, int KG, bool FP8 = false, bool SILU = false>
__global__ void __launch_bounds__(WM* WN * KG * 64, 1)
    gemm_add_rmsnorm_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bp,
                            float* __restrict__ R, const float* __restrict__ w,
                            uint16_t* __restrict__ out, unsigned long long* __restrict__ slots,
                            unsigned* __restrict__ sync, int M, int N, int K, int tiles_m,
                            int tiles_n, int rows_per_round, float eps, int gemma,
                            unsigned fault_mask, unsigned spin_limit,
                            unsigned long long* __restrict__ pwords,
                            unsigned long long slot_words, unsigned long long pword_words,
                            unsigned* __restrict__ host_flag, const float* __restrict__ x_scales,
                            int scale_rows, int scale_row0, const float* __restrict__ w_scale) {
  // Main loop: KG groups of WM x WN waves (wave tiles BM/WM x BN/WN, TM x TN MFMA blocks).
  // Epilogue: after the groups' partials are combined, EWM x WN waves, each owning a
  // BM/EWM x BN/WN tile (ETM x TN blocks).
  constexpr int GW = WM * WN;
  constexpr int NW = GW * KG;
  constexpr int TM = BM / WM / 32;
  constexpr int EWM = WM * KG;
  constexpr int WTM = BM / EWM;  // epilogue wave tile rows
  constexpr int WTN = BN / WN;
  constexpr int ETM = WTM / 32;
  constexpr int TN = WTN / 32;
  constexpr int HS = stage_halves(KG, NW);  // 32-deep halves per stage of the main loop
  constexpr int STAGE = HS * ((SILU ? 2 * BM : BM) + BN) * kBK * 2;
  static_assert(NB >= 3, "the norm epilogue uses the third ring buffer");
  static_assert((BM * WN + 2 * BM + 4) * 4 <= STAGE, "row partials fit in one stage buffer");
  char* const sb0 = ring_buffer<0, STAGE, BM, BN, NB, WM, WN>();
  char* const sb1 = ring_buffer<1, STAGE, BM, BN, NB, WM, WN>();
  float* const sred = reinterpret_cast<float*>(ring_buffer<2, STAGE, BM, BN, NB, WM, WN>());
  float* const sinv = sred + BM * WN;
  int* const sflag = reinterpret_cast<int*>(sinv + BM);
  float* const sscl = sinv + BM + 4;  // FP8: the tile's per-row dequantisation scales
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kgrp = KG == 1 ? 0 : wave / GW;  // K group of the main loop
  const int wm = ((KG == 1 ? wave : wave % GW) / WN) * KG + kgrp;  // epilogue row block
  const int wn = wave % WN;
  const float g0 = gemma ? 1.0f : 0.0f;
  const unsigned epoch = launch_epoch(sync);
  const unsigned read_epoch = epoch ^ fault_mask;  // fault_mask != 0: every wait gives up

  constexpr int EP_LD = WTN + 4;
  constexpr int EP_BYTES = 16 * EP_LD * 4;
  constexpr int EP_PER_BUF = STAGE / EP_BYTES;
  static_assert(NW <= 2 * EP_PER_BUF, "epilogue staging must fit in two stage buffers");
  constexpr int LPR = WTN / 4;   // lanes per staged row (8 or 16: one DPP row or half-row)
  constexpr int RPI = 64 / LPR;  // rows per staged read
  constexpr int NR = 16 / RPI;   // staged reads per 16-row slice
  constexpr int KEEP = ETM * 2 * NR;              // float4 of r + y per lane
  // Residual loaded before the main loop when it fits: 64 registers per lane with two waves
  // per SIMD (256 registers each), 128 with one wave per SIMD (512).
  constexpr bool PREFETCH = KG == 1 && KEEP <= (NW == 4 ? 32 : 16);
  constexpr int TPR = NW * 64 / BM;               // threads per row for the slot reads
  static_assert(TPR >= 1 && TPR <= WN, "slot-read partials reuse the row-partial buffer");
  static_assert(KG == 1 || TM % 2 == 0, "K groups hand over half of their rows");

  for (int round = 0; round * rows_per_round < tiles_m; ++round) {
    const int rows_here = min(rows_per_round, tiles_m - round * rows_per_round);
    const int count = rows_here * tiles_n;
    if ((int)blockIdx.x >= count) continue;  // uniform over the workgroup
    int tm, tn;
    constexpr int XG = 2;  // XCDs per tile row
    if ((rows_here * XG) % kNumXCDs == 0 && tiles_n % XG == 0) {
      // Each pair of XCDs computes whole tile rows, each XCD half of every row's columns
      // (workgroup b runs on XCD b % 8): a row's tiles finish together, an XCD that runs
      // slower delays only its pair's rows, and each XCD reads half of the weight.  The pairs
      // are {0, 2}, {4, 6}, {1, 3}, {5, 7}: under MFMA load the odd-numbered XCDs ran a 3-7%
      // lower clock than the even ones in every measurement on MI355X (in-kernel clock
      // stamps on three GPUs), so like is paired with like and the faster pairs do not wait
      // for a slower partner (their rows then finish, and write, before the slower pairs' do).
      const int xcd = blockIdx.x % kNumXCDs;
      const int rows_g = rows_here * XG / kNumXCDs;   // tile rows of this XCD pair
      const int cols_x = tiles_n / XG;                // column tiles per XCD
      const int j = blockIdx.x / kNumXCDs;             // 0 .. rows_g * cols_x - 1
      const int pair = ((xcd & 1) << 1) | (xcd >> 2);  // 0 .. 3
      const int member = (xcd >> 1) & 1;               // which half of the row's columns
      tm = pair * rows_g + j / cols_x;
      tn = member * cols_x + j % cols_x;
    } else {
      tile_coords(xcd_logical(blockIdx.x, count), rows_here, tiles_n, &tm, &tn);
    }
    tm += round * rows_per_round;
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    PR_PHASE(0);

    // Lane position in the staged layout: row lrow + RPI * rr of each 16-row slice, columns
    // rcol .. rcol+3 of the wave's WTN (lane id l).
    auto rcol_of = [](int l) { return (l % LPR) * 4; };
    auto row_of = [&](int l, int i, int h, int rr) {
      return wm * WTM + i * 32 + h * 16 + rr * RPI + l / LPR;
    };

    // The residual, loaded before the main loop so that its read overlaps the MFMA work (when
    // PREFETCH), else one 16-row slice ahead in the epilogue.
    float4 keep[KEEP];
    if constexpr (PREFETCH) {
      const int pcol = n0 + wn * WTN + rcol_of(lane);
#pragma unroll
      for (int i = 0; i < ETM; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int rr = 0; rr < NR; ++rr) {
            const int row = min(m0 + row_of(lane, i, h, rr), M - 1);
            keep[(i * 2 + h) * NR + rr] =
                *reinterpret_cast<const float4*>(R + (long long)row * N + pcol);
          }
    }

    // Two K groups: the last refills read one line (1.9% faster on o_proj in an interleaved
    // A/B); with one K group the tail's branch in every step cost 2-5% on 256 x 256 tiles.
    constexpr int LPW_ = HS * ((BM + BN) * kBK * 2 / 1024 / NW);
    using TailT = std::conditional_t<(FP8 || SILU || KG == 1), NoTail, ThinTail<LPW_>>;
    const TailT tail_hook{};
    const TileAcc<TM, TN> part_acc = tile_mainloop<BM, BN, NB, WM, WN, KG, TailT, FP8, SILU>(
        A, Bp, M, N, K, m0, n0, 0, FP8 ? K / (2 * kBK * KG) : K / (kBK * HS), tail_hook);
    // The ring's trailing refills (direct-to-LDS loads) have landed and every wave is past its
    // last fragment read before the stage buffers are reused below.
    __builtin_amdgcn_s_waitcnt(PR_VMCNT(0));
    __syncthreads();
    PR_PHASE(1);
    // The epilogue's per-lane offsets are formed here, from an opaque copy of the lane id, so
    // that they are not hoisted out of the round loop and kept live across the main loop.
    int el = lane;
    asm volatile("" : "+v"(el));
    const int rcol = rcol_of(el);
    const int lrow = el / LPR;
    const int col = n0 + wn * WTN + rcol;
    float* ep = reinterpret_cast<float*>((wave < EP_PER_BUF ? sb0 : sb1) +
                                         (wave % EP_PER_BUF) * EP_BYTES);
    auto load_slice = [&](int sl) {
#pragma unroll
      for (int rr = 0; rr < NR; ++rr) {
        const int row = min(m0 + row_of(el, sl >> 1, sl & 1, rr), M - 1);
        keep[sl * NR + rr] = *reinterpret_cast<const float4*>(R + (long long)row * N + col);
      }
    };
    // The first slice of the residual is in flight during the K groups' hand-over (2.5%
    // faster on o_proj than issuing it after the hand-over, equal on 256 x 256 tiles).
    if constexpr (!PREFETCH) load_slice(0);
    TileAcc<ETM, TN> tacc;
    if constexpr (KG == 1) {
      tacc = part_acc;
    } else {
      // Waves w and w + GW computed the same wave tile over the two halves of K.  Each hands
      // the other half of its rows to its partner through LDS (one 16-byte store per lane and
      // block element group) and adds the partner's half to the rows it keeps: group 0 keeps
      // the upper half, group 1 the lower.  The two-term sum is the same in either order.
      constexpr int RB = ETM * TN * 16 * 64 * 4;  // bytes handed over per wave
      constexpr int PER = STAGE / RB;             // regions per ring buffer
      static_assert(PER >= 1 && NB * PER >= NW, "hand-over regions fit in the ring");
      auto region = [&](int w) -> float4* {
        char* b = w / PER == 0 ? sb0
                               : (w / PER == 1 ? sb1
                                               : ring_buffer<2, STAGE, BM, BN, NB, WM, WN>());
        return reinterpret_cast<float4*>(b + (w % PER) * RB);
      };
      static_assert(NW <= 3 * PER, "hand-over regions use the first three ring buffers");
      float4* mine = region(wave);
      const float4* theirs = region(wave < GW ? wave + GW : wave - GW);
      auto hand_over = [&](int i0) {
#pragma unroll
        for (int i = 0; i < ETM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
              mine[((i * TN + j) * 4 + e4) * 64 + lane] =
                  make_float4(part_acc.v[i0 + i][j][4 * e4], part_acc.v[i0 + i][j][4 * e4 + 1],
                              part_acc.v[i0 + i][j][4 * e4 + 2], part_acc.v[i0 + i][j][4 * e4 + 3]);
      };
      auto combine = [&](int i0) {
#pragma unroll
        for (int i = 0; i < ETM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
              const float4 o = theirs[((i * TN + j) * 4 + e4) * 64 + lane];
              tacc.v[i][j][4 * e4] = part_acc.v[i0 + i][j][4 * e4] + o.x;
              tacc.v[i][j][4 * e4 + 1] = part_acc.v[i0 + i][j][4 * e4 + 1] + o.y;
              tacc.v[i][j][4 * e4 + 2] = part_acc.v[i0 + i][j][4 * e4 + 2] + o.z;
              tacc.v[i][j][4 * e4 + 3] = part_acc.v[i0 + i][j][4 * e4 + 3] + o.w;
            }
      };
      if (kgrp == 0) hand_over(ETM); else hand_over(0);
      __syncthreads();
      if (kgrp == 0) combine(0); else combine(ETM);
      __syncthreads();  // hand-over regions read before the epilogue reuses the buffers
    }
    PR_PHASE(2);
    if constexpr (FP8) {
      // One scale per tile row: the row's activation-group scale times the weight scale (in the
      // third ring buffer, after the K groups' hand-over has released it).
      if (threadIdx.x < BM) {
        const int row = min(m0 + (int)threadIdx.x, M - 1);
        sscl[threadIdx.x] = x_scales[(scale_row0 + row) / scale_rows] * w_scale[0];
      }
      __syncthreads();
    }
    const auto& acc = tacc.v;

#pragma unroll
    for (int i = 0; i < ETM; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (!PREFETCH)
          if (i * 2 + h + 1 < ETM * 2) load_slice(i * 2 + h + 1);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 8 * h; e < 8 * h + 8; ++e)
            ep[(((e >> 2) - 2 * h) * 8 + (el >> 5) * 4 + (e & 3)) * EP_LD + j * 32 +
               (el & 31)] = acc[i][j][e];
        __builtin_amdgcn_s_waitcnt(PR_LGKMCNT0);
#pragma unroll
        for (int rr = 0; rr < NR; ++rr) {
          const int trow = row_of(el, i, h, rr);
          const int r_in = rr * RPI + lrow;
          const int row = min(m0 + trow, M - 1);  // rows past M are computed, never stored
          float4 y = *reinterpret_cast<const float4*>(ep + r_in * EP_LD + rcol);
          if constexpr (FP8) {
            const float sc = sscl[trow];
            y = make_float4(y.x * sc, y.y * sc, y.z * sc, y.w * sc);
          }
          const float4 rv = keep[(i * 2 + h) * NR + rr];
          const float4 v = make_float4(rv.x + y.x, rv.y + y.y, rv.z + y.z, rv.w + y.w);
          // r + y stays in registers; the residual is stored with the output, after the row
          // wait, so a tile whose wait gives up leaves its residual rows as they were.
          keep[(i * 2 + h) * NR + rr] = v;
          const float q = lane_group_sum<LPR>(v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w);
          if (el % LPR == 0) sred[trow * WN + wn] = q;
        }
        __builtin_amdgcn_s_waitcnt(PR_LGKMCNT0);  // reads done before the next slice
      }
    }
    __syncthreads();
    PR_PHASE(3);
    const unsigned long long tag = (unsigned long long)epoch << 32;
    if (threadIdx.x < BM) {
      float p = 0.0f;
#pragma unroll
      for (int q = 0; q < WN; ++q) p += sred[threadIdx.x * WN + q];
      const int row = m0 + threadIdx.x;
      if (row < M)
        __hip_atomic_store(slots + (long long)tn * M + row, tag | __float_as_uint(p),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned* cnt = sync + 3 + tm;
      __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      PR_PHASE(4);
      unsigned polls = 0;
      while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                 (unsigned)tiles_n &&
             polls++ < spin_limit)
        __builtin_amdgcn_s_sleep(1);
      *sflag = 1;
      PR_PHASE(5);
    }
    __syncthreads();
    {
      // The row's slots in tile-column order: TPR threads per row each add a contiguous run
      // of ceil(tiles_n / TPR) slots (up to 16 loads in flight per batch), then the runs are
      // added in order.
      const int trow = threadIdx.x % BM;
      const int part = threadIdx.x / BM;
      const int row = m0 + trow;
      const int per = (tiles_n + TPR - 1) / TPR;
      const int q_begin = min(part * per, tiles_n), q_end = min(q_begin + per, tiles_n);
      float ss = 0.0f;
      if (row < M) {
        const unsigned long long* ps = slots + row;  // slot q at ps[q * M]
        unsigned polls = 0;  // one budget for the whole run
        for (int q0 = q_begin; q0 < q_end; q0 += 16) {
          unsigned long long sv[16];
#pragma unroll
          for (int u = 0; u < 16; ++u)
            sv[u] = q0 + u < q_end ? __hip_atomic_load(ps + (long long)(q0 + u) * M,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                   : (unsigned long long)read_epoch << 32;
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            while ((sv[u] >> 32) != read_epoch) {
              if (polls++ >= spin_limit) {
                *sflag = 0;  // the tile gives up
                break;
              }
              __builtin_amdgcn_s_sleep(1);
              sv[u] = __hip_atomic_load(ps + (long long)(q0 + u) * M, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
            }
            if (q0 + u < q_end) ss += __uint_as_float((unsigned)sv[u]);
          }
        }
      }
      sred[trow * TPR + part] = ss;
    }
    __syncthreads();
    PR_PHASE(6);
    if (threadIdx.x < BM && m0 + threadIdx.x < M) {
      float ss = 0.0f;
#pragma unroll
      for (int q = 0; q < TPR; ++q) ss += sred[threadIdx.x * TPR + q];
      sinv[threadIdx.x] = 1.0f / sqrtf(ss / (float)N + eps);
    }
    __syncthreads();
    if (*sflag == 0) {
      if (threadIdx.x == 0) report_give_up(sync, host_flag);
    } else {
      const float4 g = *reinterpret_cast<const float4*>(w + col);
      const float gx = g.x + g0, gy = g.y + g0, gz = g.z + g0, gw = g.w + g0;
      // Tiles narrower than 256 columns store at device scope (sc1): the lines go through the
      // XCD's L2 to memory as they are written, so the launch's end has fewer dirty lines to
      // write back.  256x256 tiles, whose rows finish further apart, keep streaming stores.
      constexpr bool kDeviceScopeStores = BN < 256;
      const int vrows = min(BM, M - m0);
      const __amdgpu_buffer_rsrc_t rs_r = __builtin_amdgcn_make_buffer_rsrc(
          R + (long long)m0 * N, 0, vrows * N * 4, kBufferRsrcWord3);
      const __amdgpu_buffer_rsrc_t rs_o = __builtin_amdgcn_make_buffer_rsrc(
          out + (long long)m0 * N, 0, vrows * N * 2, kBufferRsrcWord3);
#pragma unroll
      for (int i = 0; i < ETM; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int rr = 0; rr < NR; ++rr) {
            const int trow = row_of(el, i, h, rr);
            const int row = m0 + trow;
            if (row < M) {
              const float4 v = keep[(i * 2 + h) * NR + rr];
              // The updated residual and the output are not read again here.
              if constexpr (kDeviceScopeStores)
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4_t, f32x4_t{v.x, v.y, v.z, v.w}), rs_r,
                    (trow * N + col) * 4, 0, kStoreSc1);
              else
                __builtin_nontemporal_store(
                    f32x4_t{v.x, v.y, v.z, v.w},
                    reinterpret_cast<f32x4_t*>(R + (long long)row * N + col));
              const float inv = sinv[trow];
              const uint32_t o0 = f32_to_bf16_rne(v.x * inv * gx);
              const uint32_t o1 = f32_to_bf16_rne(v.y * inv * gy);
              const uint32_t o2 = f32_to_bf16_rne(v.z * inv * gz);
              const uint32_t o3 = f32_to_bf16_rne(v.w * inv * gw);
              if constexpr (kDeviceScopeStores)
                __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{o0 | (o1 << 16), o2 | (o3 << 16)},
                                                      rs_o, (trow * N + col) * 2, 0, kStoreSc1);
              else
                __builtin_nontemporal_store(
                    (unsigned long long)(o0 | (o1 << 16)) |
                        ((unsigned long long)(o2 | (o3 << 16)) << 32),
                    reinterpret_cast<unsigned long long*>(out + (long long)row * N + col));
            }
          }
    }
    PR_PHASE(7);
    __syncthreads();  // LDS is refilled by the next tile's prologue
  }

  // The last workgroup to finish returns the counters to zero for the next launch (every
  // other workgroup is past its last counter read by then).
  if (threadIdx.x == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *sflag = prev == gridDim.x - 1;
  }
  __syncthreads();
  if (*sflag) finish_launch(sync, tiles_m, epoch, slots, slot_words, pwords, pword_words);
}

// --------------------------------------------------------------------------------------------
// Single launch with the K range of each 256 x 256 tile split over a pair of workgroups.
//
// When a shape has fewer 256 x 256 tiles than the GPU has CUs, a workgroup pair shares each
// tile: workgroup h (0 or 1) runs the main loop over K half h, so every CU works on a large
// tile (fewer operand bytes per flop than a 256 x 128 tile over the whole K).  The pair then
// swaps partial sums: h keeps tile rows [128 h, 128 h + 128) and hands the other 128 rows'
// partial to its partner through an exchange region, announced by an epoch-tagged ready word
// stored after the writes have completed.  The pair normally sits on one XCD (workgroups b
// and b ^ 8); each workgroup publishes its XCD id when its round starts, and a writer that
// finds its partner's id (with this launch's epoch) equal to its own writes the region with
// plain stores, which land in the XCD's shared L2, and says so in its ready word; the reader
// then drops its own L1 copy of any earlier round's region and reads with plain loads from
// that L2.  Otherwise both sides use device-scope accesses, which reach the memory-side
// coherence point, so the exchange is correct wherever the pair runs.  Each workgroup adds
// the two partials of its rows
// (a two-term fp32 sum, the same in either order) and runs the residual add and RMSNorm of
// its 128 x 256 block with the row-partial slot protocol of gemm_add_rmsnorm_kernel: its block
// row has tiles_n column tiles, one slot per row and column tile, and one counter per
// 128-row block.
//
// The main loop's last four ring refills load the kept rows' residual into LDS (one 1 KiB row
// per load, the loads a stage would take), so it lands while the last stages compute.  After
// the loop the four waves that hand their rows over write the hand-over; the four waves that
// keep their rows add the partner's partial, form r + y in place in LDS and the row sums; all
// eight waves then wait for the row block and write the residual and the output from LDS.
//
// Exchange regions: `xbuf` holds 128 KiB per workgroup and round parity (the region a
// workgroup writes in round q is rewritten in round q + 2 only after the partner's round q + 1
// ready word, i.e. after the partner finished reading it).  pwords: four 64-bit words per tile
// of the launch, per half h the XCD-id word [4 t + 2 h] and the ready word [4 t + 2 h + 1],
// each {epoch of the launch that wrote it, value}.
// --------------------------------------------------------------------------------------------
// Tail hook of the pair form: the main loop's last NB - 1 refills load the kept rows'
// residual instead of re-reading the last stage.  Refill j brings kept rows [32 j, 32 j + 32)
// (1 KiB rows of 256 fp32 columns), four rows per wave, into the buffer it refills.
struct ResidualTail {
  static constexpr int kLoads = 4;
  const float* R;
  int N, n0, row0, M, wave;
  uint32_t lane_off;
  __device__ void operator()(int j, char* buf) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int row = row0 + 32 * j + 4 * wave + i;
      row = row < M ? row : M - 1;  // rows past M are computed, never stored
      load_to_lds16(reinterpret_cast<const char*>(R + (long long)row * N + n0), lane_off,
                    buf + (4 * wave + i) * 1024);
    }
  }
};

template <int NB>
__global__ void __launch_bounds__(512, 1)
    gemm_add_rmsnorm_pair_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bp,
                                 float* __restrict__ R, const float* __restrict__ w,
                                 uint16_t* __restrict__ out, unsigned long long* __restrict__ slots,
                                 unsigned* __restrict__ sync,
                                 unsigned long long* __restrict__ pwords,
                                 unsigned long long* __restrict__ xbuf, int M, int N, int K,
                                 int tiles_m, int tiles_n, int rows_per_round, float eps,
                                 int gemma, unsigned fault_mask, unsigned spin_limit,
                                 unsigned long long slot_words,
                                 unsigned long long pword_words,
                                 unsigned* __restrict__ host_flag) {
  constexpr int BM = 256, BN = 256, WM = 2, WN = 4;
  constexpr int TM = 4, TN = 2;       // 128 x 64 wave tiles
  constexpr int HB = 128;             // rows kept per workgroup
  constexpr int STAGE = (BM + BN) * kBK * 2;  // 32 KiB
  constexpr int XW = TM * TN * 8 * 64;        // 64-bit exchange words per wave (32 KiB)
  static_assert(NB == 5 && STAGE == 32 * 1024, "four residual buffers and a staging buffer");
  constexpr int EP_LD = 64 + 4;
  constexpr int EP_BYTES = 16 * EP_LD * 4;
  static_assert(4 * EP_BYTES + (HB * WN + HB + 3) * 4 <= STAGE, "staging fits in buffer 4");
  // The main loop's last refills bring the kept rows' residual: block j (32 rows) lands in
  // ring buffer (nk + j) % NB, and the buffer of the last stage, (nk - 1) % NB, is the staging
  // buffer of the epilogue.  Buffers are separate LDS objects, chosen by a uniform index.
  const int nk = K / 2 / kBK;  // >= NB - 1 (K >= 256), so the last NB - 1 steps are tail refills
  auto ringbuf = [](int u) -> char* {
    char* const b0 = ring_buffer<0, STAGE, BM, BN, NB, WM, WN>();
    char* const b1 = ring_buffer<1, STAGE, BM, BN, NB, WM, WN>();
    char* const b2 = ring_buffer<2, STAGE, BM, BN, NB, WM, WN>();
    char* const b3 = ring_buffer<3, STAGE, BM, BN, NB, WM, WN>();
    char* const b4 = ring_buffer<4, STAGE, BM, BN, NB, WM, WN>();
    return u == 0 ? b0 : (u == 1 ? b1 : (u == 2 ? b2 : (u == 3 ? b3 : b4)));
  };
  auto rbuf = [&](int j) -> char* { return ringbuf((nk + j) % NB); };
  char* const sb4 = ringbuf((nk + NB - 1) % NB);
  float* const sred = reinterpret_cast<float*>(sb4 + 4 * EP_BYTES);
  float* const sinv = sred + HB * WN;
  int* const sflag = reinterpret_cast<int*>(sinv + HB);
  int* const smode = sflag + 1;  // this workgroup writes its hand-over with plain stores
  int* const spart = sflag + 2;  // the partner wrote its hand-over with plain stores
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;
  const float g0 = gemma ? 1.0f : 0.0f;
  const unsigned epoch = launch_epoch(sync);
  const unsigned read_epoch = epoch ^ fault_mask;  // fault_mask != 0: every wait gives up

  for (int round = 0; round * rows_per_round < tiles_m; ++round) {
    const int rows_here = min(rows_per_round, tiles_m - round * rows_per_round);
    const int tiles = rows_here * tiles_n;
    const int count = 2 * tiles;
    if ((int)blockIdx.x >= count) continue;  // uniform over the workgroup
    // Pairs: workgroups b and b ^ 8 (same XCD, b % 8) within each group of 16, else b and
    // b ^ 1.  q numbers the tiles so that q % 8 is the pair's XCD.
    const int b = blockIdx.x;
    const int full = count / 16 * 16;
    int h, q, partner;
    if (b < full) {
      h = (b >> 3) & 1;
      q = (b >> 4) * 8 + (b & 7);
      partner = b ^ 8;
    } else {
      h = b & 1;
      q = b >> 1;
      partner = b ^ 1;
    }
    int tm, tn;
    if (full == count && (rows_here * 2) % kNumXCDs == 0 && tiles_n % 2 == 0) {
      // Each pair of XCDs computes whole tile rows, each XCD half of every row's columns.
      const int xcd = q % kNumXCDs;
      const int rows_g = rows_here * 2 / kNumXCDs;
      const int cols_x = tiles_n / 2;
      const int j = q / kNumXCDs;
      tm = (xcd / 2) * rows_g + j / cols_x;
      tn = (xcd % 2) * cols_x + j % cols_x;
    } else {
      tile_coords(xcd_logical(q, tiles), rows_here, tiles_n, &tm, &tn);
    }
    tm += round * rows_per_round;
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int own0 = m0 + h * HB;  // first row this workgroup normalises
    const int tile_id = tm * tiles_n + tn;
    unsigned long long* const my_words = pwords + tile_id * 4 + h * 2;
    const unsigned long long* const partner_words = pwords + tile_id * 4 + (1 - h) * 2;
    unsigned xcc = 0;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    xcc &= 0xff;
    const unsigned long long tag = (unsigned long long)epoch << 32;
    if (threadIdx.x == 0)
      __hip_atomic_store(my_words, tag | xcc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    const ResidualTail rtail{R, N, n0, own0, M, wave, (uint32_t)lane * 16u};
    TileAcc<TM, TN> acc = tile_mainloop<BM, BN, NB, WM, WN, 1, ResidualTail>(
        A, Bp, M, N, K, m0, n0, h * (K / 2), nk, rtail);
    // Plain hand-over only if the partner's id word is this launch's and names this XCD.
    unsigned long long pid = 0;
    if (threadIdx.x == 0)
      pid = __hip_atomic_load(partner_words, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(PR_VMCNT(0));
    __syncthreads();  // the ring is free
    if (threadIdx.x == 0) *smode = pid == (tag | xcc);
    __syncthreads();
    const bool plain = *smode != 0;
    // Lane-dependent epilogue offsets come from an opaque copy of the lane id, so that they are
    // formed here rather than hoisted out of the round loop and kept live across the main loop.
    int el = lane;
    asm volatile("" : "+v"(el));
    int et = threadIdx.x;
    asm volatile("" : "+v"(et));

    unsigned long long* const xmine = xbuf + (size_t)((round & 1) * gridDim.x + b) * (4 * XW);
    const unsigned long long* const xpart =
        xbuf + (size_t)((round & 1) * gridDim.x + partner) * (4 * XW);
    if (wm != h) {
      // Hand over this wave's rows (the partner keeps them): 16-byte plain stores (same XCD)
      // or 8-byte device-scope stores, each in its own layout.
      if (plain) {
        float4* xw = reinterpret_cast<float4*>(xmine + wn * XW);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
              xw[((i * TN + j) * 4 + e4) * 64 + el] =
                  make_float4(acc.v[i][j][4 * e4], acc.v[i][j][4 * e4 + 1],
                              acc.v[i][j][4 * e4 + 2], acc.v[i][j][4 * e4 + 3]);
      } else {
        unsigned long long* xw = xmine + wn * XW;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) {
              const unsigned long long v =
                  (unsigned long long)__float_as_uint(acc.v[i][j][2 * e2]) |
                  ((unsigned long long)__float_as_uint(acc.v[i][j][2 * e2 + 1]) << 32);
              __hip_atomic_store(xw + ((i * TN + j) * 8 + e2) * 64 + el, v, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
            }
      }
      __builtin_amdgcn_s_waitcnt(PR_VMCNT(0));  // hand-over written
    }
    __syncthreads();
    if (et == 0) {
      __hip_atomic_store(my_words + 1, tag | (plain ? 1u : 0u), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      unsigned polls = 0;
      int ok = 1;
      unsigned long long v;
      while (((v = __hip_atomic_load(partner_words + 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT)) >> 32) != read_epoch) {
        if (polls++ >= spin_limit) {
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      *sflag = ok;
      *spart = (int)(v & 1);
    }
    __syncthreads();
    if (*sflag == 0) {
      // The partner never announced its half: this block writes nothing (its row block's
      // waits give up in turn).
      if (et == 0) report_give_up(sync, host_flag);
      __syncthreads();
      continue;
    }

    const int lrow = el / 16;        // staged layout: 16 lanes per row, 4 floats each
    const int rcol = (el % 16) * 4;
    if (wm == h && *spart) {
      // The partner's partial of the kept rows, from this XCD's L2: 16-byte loads after
      // dropping any L1 copy of the region (it may hold an earlier round's contents).
      asm volatile("buffer_inv sc0" ::: "memory");
      const float4* xp = reinterpret_cast<const float4*>(xpart + wn * XW);
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        float4 pv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) pv[u] = xp[(part * 16 + u) * 64 + el];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int idx = part * 16 + u;  // (i * TN + j) * 4 + e4
          const int i = idx / (TN * 4), j = (idx / 4) % TN, e4 = idx % 4;
          acc.v[i][j][4 * e4] += pv[u].x;
          acc.v[i][j][4 * e4 + 1] += pv[u].y;
          acc.v[i][j][4 * e4 + 2] += pv[u].z;
          acc.v[i][j][4 * e4 + 3] += pv[u].w;
        }
      }
    } else if (wm == h) {
      // The partner's partial through the memory-side coherence point (batches of 16 loads).
      const unsigned long long* xp = xpart + wn * XW;
#pragma unroll
      for (int part = 0; part < 4; ++part) {
        unsigned long long pv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          pv[u] = __hip_atomic_load(xp + (part * 16 + u) * 64 + el, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int idx = part * 16 + u;  // (i * TN + j) * 8 + e2
          const int i = idx / (TN * 8), j = (idx / 8) % TN, e2 = idx % 8;
          acc.v[i][j][2 * e2] += __uint_as_float((unsigned)pv[u]);
          acc.v[i][j][2 * e2 + 1] += __uint_as_float((unsigned)(pv[u] >> 32));
        }
      }
    }
    if (wm == h) {
      // r + y in place in LDS, and per-row sums of squares of this wave's 64 columns.
      float* ep = reinterpret_cast<float*>(sb4 + wn * EP_BYTES);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 8 * hh; e < 8 * hh + 8; ++e)
              ep[(((e >> 2) - 2 * hh) * 8 + (el >> 5) * 4 + (e & 3)) * EP_LD + j * 32 +
                 (el & 31)] = acc.v[i][j][e];
          __builtin_amdgcn_s_waitcnt(PR_LGKMCNT0);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int r_in = rr * 4 + lrow;
            const int trow = i * 32 + hh * 16 + r_in;  // row within the kept 128 (buffer i)
            const float4 y = *reinterpret_cast<const float4*>(ep + r_in * EP_LD + rcol);
            float4* rp = reinterpret_cast<float4*>(rbuf(i) + (trow % 32) * 1024 +
                                                   (wn * 64 + rcol) * 4);
            const float4 rv = *rp;
            const float4 v = make_float4(rv.x + y.x, rv.y + y.y, rv.z + y.z, rv.w + y.w);
            *rp = v;
            const float sq = lane_group_sum<16>(v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w);
            if (el % 16 == 0) sred[trow * WN + wn] = sq;
          }
          __builtin_amdgcn_s_waitcnt(PR_LGKMCNT0);  // reads done before the next slice
        }
      }
    }
    __syncthreads();
    if (et < HB) {
      float p = 0.0f;
#pragma unroll
      for (int c = 0; c < WN; ++c) p += sred[et * WN + c];
      const int row = own0 + et;
      if (row < M)
        __hip_atomic_store(slots + (long long)tn * M + row, tag | __float_as_uint(p),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    unsigned* const cnt = sync + 3 + tm * 2 + h;
    if (et == 0) {
      __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      unsigned polls = 0;
      while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                 (unsigned)tiles_n &&
             polls++ < spin_limit)
        __builtin_amdgcn_s_sleep(1);
      *sflag = 1;
    }
    __syncthreads();
    {
      // The row block's slots in tile-column order: four threads per row, each a contiguous
      // run of ceil(tiles_n / 4) slots, then the runs in order.
      const int trow = et % HB;
      const int part = et / HB;
      const int row = own0 + trow;
      const int per = (tiles_n + 3) / 4;
      const int c_begin = min(part * per, tiles_n), c_end = min(c_begin + per, tiles_n);
      float ss = 0.0f;
      if (row < M) {
        const unsigned long long* ps = slots + row;
        unsigned polls = 0;
        unsigned long long sv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          sv[u] = c_begin + u < c_end ? __hip_atomic_load(ps + (long long)(c_begin + u) * M,
                                                          __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT)
                                      : (unsigned long long)read_epoch << 32;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          while ((sv[u] >> 32) != read_epoch) {
            if (polls++ >= spin_limit) {
              *sflag = 0;  // the block gives up
              break;
            }
            __builtin_amdgcn_s_sleep(1);
            sv[u] = __hip_atomic_load(ps + (long long)(c_begin + u) * M, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
          }
          if (c_begin + u < c_end) ss += __uint_as_float((unsigned)sv[u]);
        }
      }
      sred[trow * 4 + part] = ss;  // the publish reads of sred are two barriers back
    }
    __syncthreads();
    if (et < HB && own0 + et < M) {
      const float ss = ((sred[et * 4] + sred[et * 4 + 1]) +
                        sred[et * 4 + 2]) + sred[et * 4 + 3];
      sinv[et] = 1.0f / sqrtf(ss / (float)N + eps);
    }
    __syncthreads();
    if (*sflag == 0) {
      if (et == 0) report_give_up(sync, host_flag);
    } else {
      // The updated residual (16 rows of 1 KiB per wave, from LDS), stored only now so that a
      // block whose wait gave up leaves its residual rows as they were.
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int trow = wave * 16 + k;
        const int row = own0 + trow;
        const float4 v = *reinterpret_cast<const float4*>(rbuf(trow / 32) + (trow % 32) * 1024 +
                                                          el * 16);
        if (row < M)
          __builtin_nontemporal_store(f32x4_t{v.x, v.y, v.z, v.w},
                                      reinterpret_cast<f32x4_t*>(R + (long long)row * N + n0 +
                                                                 el * 4));
      }
      // Output: 16 rows per wave, two rows per instruction, 8 columns (16 bytes) per lane.
      const int c8 = (el & 31) * 8;
      const float4 ga = *reinterpret_cast<const float4*>(w + n0 + c8);
      const float4 gb = *reinterpret_cast<const float4*>(w + n0 + c8 + 4);
      const float gx[8] = {ga.x + g0, ga.y + g0, ga.z + g0, ga.w + g0,
                           gb.x + g0, gb.y + g0, gb.z + g0, gb.w + g0};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int trow = wave * 16 + k * 2 + (el >> 5);
        const int row = own0 + trow;
        if (row < M) {
          const float* src =
              reinterpret_cast<const float*>(rbuf(trow / 32) + (trow % 32) * 1024) + c8;
          const float4 va = *reinterpret_cast<const float4*>(src);
          const float4 vb = *reinterpret_cast<const float4*>(src + 4);
          const float inv = sinv[trow];
          const float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
          uint32_t o[4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            o[t] = f32_to_bf16_rne(v[2 * t] * inv * gx[2 * t]) |
                   (f32_to_bf16_rne(v[2 * t + 1] * inv * gx[2 * t + 1]) << 16);
          __builtin_nontemporal_store(
              u32x4_t{o[0], o[1], o[2], o[3]},
              reinterpret_cast<u32x4_t*>(out + (long long)row * N + n0 + c8));
        }
      }
    }
    __syncthreads();  // LDS is refilled by the next tile's prologue
  }

  // The last workgroup to finish returns the counters to zero for the next launch.
  if (threadIdx.x == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *sflag = prev == gridDim.x - 1;
  }
  __syncthreads();
  if (*sflag) finish_launch(sync, 2 * tiles_m, epoch, slots, slot_words, pwords, pword_words);
}

// --------------------------------------------------------------------------------------------
// Residual add + RMSNorm: one wavefront per row, the row held in registers (NV float4 per lane,
// H = 256 * NV).  Loads of the whole row are issued before any use so that each wave keeps
// NV * (1 + planes) 16-byte loads per lane in flight.
// --------------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float4 round_bf16_4(float4 v) {
  return make_float4(bf16_to_f32(f32_to_bf16_rne(v.x)), bf16_to_f32(f32_to_bf16_rne(v.y)),
                     bf16_to_f32(f32_to_bf16_rne(v.z)), bf16_to_f32(f32_to_bf16_rne(v.w)));
}

// Rows are split over WPR waves (WPR = 1, 2, 4, 8): wave w of a row holds the columns
// [w*H/WPR, (w+1)*H/WPR) as NV float4 per lane (H = 256 * NV * WPR).  The sum of squares is
// taken over S fixed segments of the row (S = 8, 4, 2 or 1, set by H alone): each segment's
// partial is accumulated per lane in column order and reduced across the wave, and the S
// partials are added in segment order.  That order does not depend on WPR, on how many rows
// the launch has or on timing, so a row's result is the same in a microchunk and in the whole
// batch.  A workgroup handles RPB rows at a time and strides over row groups by the grid size,
// so the launch may use fewer workgroups (CUs) than there are row groups.
template <int NV, int WPR, bool YB>
__global__ void __launch_bounds__(WPR <= 4 ? 256 : 64 * WPR)
    add_rmsnorm_kernel(const float* __restrict__ yf, const uint16_t* __restrict__ yb,
                       int nplanes, long long plane_stride, int round_y, float* __restrict__ r,
                       const float* __restrict__ w, uint16_t* __restrict__ out, int rows, int H,
                       float eps, int gemma) {
  constexpr int RPB = WPR <= 4 ? 4 / WPR : 1;  // rows per workgroup per iteration
  constexpr int N4 = NV * WPR;                   // float4 per lane over the whole row
  constexpr int S = N4 % 8 == 0 ? 8 : (N4 % 4 == 0 ? 4 : (N4 % 2 == 0 ? 2 : 1));
  static_assert(S % WPR == 0, "each wave holds whole segments");
  constexpr int SW = S / WPR;  // segments held by one wave
  constexpr int PER = NV / SW;  // float4 per lane per segment
  // Segment partials, double-buffered by iteration parity: a wave reuses a buffer two
  // iterations later, after every wave has passed the barrier of the iteration in between
  // (and so has finished reading it).
  __shared__ float part[2][RPB][S];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // row bases are uniform
  const int lane = threadIdx.x & 63;
  const int row_in = wave / WPR;
  const int wr = wave % WPR;
  const float g0 = gemma ? 1.0f : 0.0f;
  const float* wc = w + wr * (H / WPR);
  int parity = 0;
  // The loop bound depends only on blockIdx, so every wave of a workgroup takes the same trips
  // (the barrier below is uniform).
  for (int group = blockIdx.x; group * RPB < rows; group += gridDim.x, parity ^= 1) {
    // Keeps the norm-weight loads inside the loop: hoisted out of it they would hold NV more
    // float4 per lane for the whole kernel (most workgroups run one trip).
    asm volatile("" ::: "memory");
    const int row = group * RPB + row_in;
    const bool live = row < rows;
    const long long base = (long long)(live ? row : 0) * H + wr * (H / WPR);
    float4 v[NV];
    float seg[SW];
#pragma unroll
    for (int j = 0; j < SW; ++j) seg[j] = 0.0f;
    if (live) {
      // Loads go out in batches of NV independent 16-byte loads per lane (the residual, then
      // the first plane or the bf16 y, then each further plane), so each wave keeps a whole
      // batch in flight rather than one load at a time.
      float4 rv[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i)
        rv[i] = *reinterpret_cast<const float4*>(r + base + (i * 64 + lane) * 4);
      if constexpr (YB) {
        (void)yf;
        (void)nplanes;
        (void)plane_stride;
        (void)round_y;
        uint2 yv[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i)
          yv[i] = *reinterpret_cast<const uint2*>(yb + base + (i * 64 + lane) * 4);
#pragma unroll
        for (int i = 0; i < NV; ++i)
          v[i] = make_float4(rv[i].x + bf16_to_f32(yv[i].x & 0xffffu),
                             rv[i].y + bf16_to_f32(yv[i].x >> 16),
                             rv[i].z + bf16_to_f32(yv[i].y & 0xffffu),
                             rv[i].w + bf16_to_f32(yv[i].y >> 16));
      } else {
        (void)yb;
        // y = plane 0 + plane 1 + ... in plane order, then r + y.
#pragma unroll
        for (int i = 0; i < NV; ++i)
          v[i] = *reinterpret_cast<const float4*>(yf + base + (i * 64 + lane) * 4);
        for (int p = 1; p < nplanes; ++p) {
          float4 q[NV];
#pragma unroll
          for (int i = 0; i < NV; ++i)
            q[i] = *reinterpret_cast<const float4*>(yf + p * plane_stride + base +
                                                    (i * 64 + lane) * 4);
#pragma unroll
          for (int i = 0; i < NV; ++i) {
            v[i].x += q[i].x;
            v[i].y += q[i].y;
            v[i].z += q[i].z;
            v[i].w += q[i].w;
          }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          if (round_y) v[i] = round_bf16_4(v[i]);
          v[i] = make_float4(rv[i].x + v[i].x, rv[i].y + v[i].y, rv[i].z + v[i].z,
                             rv[i].w + v[i].w);
        }
      }
      // The residual and the output are stored at device scope (sc1): the lines go through the
      // L2 to memory as they are written instead of staying dirty until the launch's end.
      const __amdgpu_buffer_rsrc_t rs_r =
          __builtin_amdgcn_make_buffer_rsrc(r + base, 0, (H / WPR) * 4, kBufferRsrcWord3);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c = (i * 64 + lane) * 4;
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4_t, f32x4_t{v[i].x, v[i].y, v[i].z, v[i].w}), rs_r, c * 4, 0,
            kStoreSc1);
      }
#pragma unroll
      for (int j = 0; j < SW; ++j) {
        float a = 0.0f;
#pragma unroll
        for (int i = j * PER; i < (j + 1) * PER; ++i)
          a += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
        seg[j] = wave_sum(a);
      }
    }
    float ss = 0.0f;
    if (WPR > 1) {
      if (lane == 0) {
#pragma unroll
        for (int j = 0; j < SW; ++j) part[parity][row_in][wr * SW + j] = seg[j];
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < S; ++q) ss += part[parity][row_in][q];
    } else {
#pragma unroll
      for (int q = 0; q < S; ++q) ss += seg[q];
    }
    if (live) {
      const float inv = 1.0f / sqrtf(ss / (float)H + eps);
      const __amdgpu_buffer_rsrc_t rs_o =
          __builtin_amdgcn_make_buffer_rsrc(out + base, 0, (H / WPR) * 2, kBufferRsrcWord3);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c = (i * 64 + lane) * 4;
        const float4 g = *reinterpret_cast<const float4*>(wc + c);
        const uint32_t o0 = f32_to_bf16_rne(v[i].x * inv * (g.x + g0));
        const uint32_t o1 = f32_to_bf16_rne(v[i].y * inv * (g.y + g0));
        const uint32_t o2 = f32_to_bf16_rne(v[i].z * inv * (g.z + g0));
        const uint32_t o3 = f32_to_bf16_rne(v[i].w * inv * (g.w + g0));
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{o0 | (o1 << 16), o2 | (o3 << 16)}, rs_o,
                                              c * 2, 0, kStoreSc1);
      }
    }
  }
}

// Any H that is a multiple of 64 (and rows wider than the register-resident variants): one
// wave per row, two passes over the row, the second re-reading the just-written residual.
// Waves stride over rows by the grid size.
__global__ void __launch_bounds__(256)
    add_rmsnorm_generic_kernel(const float* __restrict__ yf, const uint16_t* __restrict__ yb,
                               int nplanes, long long plane_stride, int round_y,
                               float* __restrict__ r, const float* __restrict__ w,
                               uint16_t* __restrict__ out, int rows, int H, float eps,
                               int gemma) {
  const int lane = threadIdx.x & 63;
  const float g0 = gemma ? 1.0f : 0.0f;
  for (int row = blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += gridDim.x * 4) {
    const long long base = (long long)row * H;
    float ss = 0.0f;
    for (int c = lane; c < H; c += 64) {
      float y;
      if (yb != nullptr) {
        y = bf16_to_f32(yb[base + c]);
      } else {
        y = yf[base + c];
        for (int p = 1; p < nplanes; ++p) y += yf[p * plane_stride + base + c];
        if (round_y) y = bf16_to_f32(f32_to_bf16_rne(y));
      }
      const float v = r[base + c] + y;
      r[base + c] = v;
      ss += v * v;
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)H + eps);
    for (int c = lane; c < H; c += 64)
      out[base + c] = (uint16_t)f32_to_bf16_rne(r[base + c] * inv * (w[c] + g0));
  }
}

// --------------------------------------------------------------------------------------------
// Weight preparation: dst[((k/8)*H + h)*8 + k%8] = W[h][k].
// --------------------------------------------------------------------------------------------
__global__ void prepare_weight_out_in_kernel(const uint16_t* __restrict__ W,
                                             uint16_t* __restrict__ dst, int K, int H) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // (k-group, h)
  const long long total = (long long)(K / 8) * H;
  if (idx >= total) return;
  const int kg = (int)(idx / H);
  const int h = (int)(idx % H);
  const uint4 v = *reinterpret_cast<const uint4*>(W + (long long)h * K + kg * 8);
  *reinterpret_cast<uint4*>(dst + idx * 8) = v;
}

__global__ void prepare_weight_in_out_kernel(const uint16_t* __restrict__ Wt,
                                             uint16_t* __restrict__ dst, int K, int H) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)(K / 8) * H;
  if (idx >= total) return;
  const int kg = (int)(idx / H);
  const int h = (int)(idx % H);
  uint32_t p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = Wt[(long long)(kg * 8 + 2 * j) * H + h];
    const uint32_t hi = Wt[(long long)(kg * 8 + 2 * j + 1) * H + h];
    p[j] = lo | (hi << 16);
  }
  *reinterpret_cast<uint4*>(dst + idx * 8) = make_uint4(p[0], p[1], p[2], p[3]);
}

// --------------------------------------------------------------------------------------------
// Debug and tuning helpers.
// --------------------------------------------------------------------------------------------
__global__ void delay_kernel(int iters) {
  for (int i = 0; i < iters; ++i) __builtin_amdgcn_s_sleep(127);
}

__global__ void fill_nan_kernel(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = __uint_as_float(0x7fc00000u);
}

__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  // splitmix-style integer finaliser
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ void fill_bf16_hash_kernel(uint16_t* __restrict__ p, size_t n, uint32_t seed,
                                      float scale) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const uint32_t h = hash32((uint32_t)i * 2654435761u ^ seed ^ (uint32_t)(i >> 32));
    const float u = (float)(h >> 8) * (1.0f / 16777216.0f) * 2.0f - 1.0f;
    p[i] = (uint16_t)f32_to_bf16_rne(u * scale);
  }
}

__global__ void fill_f32_hash_kernel(float* __restrict__ p, size_t n, uint32_t seed, float scale,
                                     float offset) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const uint32_t h = hash32((uint32_t)i * 2654435761u ^ seed ^ (uint32_t)(i >> 32));
    const float u = (float)(h >> 8) * (1.0f / 16777216.0f) * 2.0f - 1.0f;
    p[i] = u * scale + offset;
  }
}

#define PR_TRY_K(call)            \
  do {                            \
    const int rc_ = (call);       \
    if (rc_ != PR_OK) return rc_; \
  } while (0)

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PR_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return PR_OK;
}

// Completion event of a launch: an event record right after it on the same stream.
int record_after(int rc, hipEvent_t done, hipStream_t s) {
  if (rc != PR_OK || done == nullptr) return rc;
  const hipError_t e = hipEventRecord(done, s);
  if (e != hipSuccess) return fail(PR_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  return PR_OK;
}

// The extended launch signals the event from the dispatch itself, which costs the host less
// than a separate record; PR_EXT_LAUNCH=0 selects launch + record.
bool ext_launch_events() {
  const char* v = std::getenv("PR_EXT_LAUNCH");
  return v == nullptr || v[0] != '0';
}

template <int BM, int BN, int NB, int WM, int WN>
int launch_gemm_t(const uint16_t* x, const uint16_t* Wp, void* C, bool bf16_out, int M, int N,
                  int K, int split, long long plane_stride, hipStream_t s, hipEvent_t done,
                  hipEvent_t t0, hipEvent_t t1) {
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const int k_len = K / split;
  const unsigned grid = (unsigned)(tiles_m * tiles_n * split);
  float* cf = bf16_out ? nullptr : static_cast<float*>(C);
  uint16_t* cb = bf16_out ? static_cast<uint16_t*>(C) : nullptr;
  if (t0 != nullptr) {
    // Timed launch: the dispatch records its own start and end; the completion event follows.
    hipExtLaunchKernelGGL((gemm_bf16_kernel<BM, BN, NB, WM, WN>), dim3(grid), dim3(WM * WN * 64),
                          0, s, t0, t1, 0, x, Wp, cf, cb, M, N, K, k_len, plane_stride, tiles_m,
                          tiles_n, split);
    return record_after(check_launch("gemm_bf16_kernel"), done, s);
  }
  if (done != nullptr && ext_launch_events()) {
    // The completion event is signalled by the dispatch itself.
    hipExtLaunchKernelGGL((gemm_bf16_kernel<BM, BN, NB, WM, WN>), dim3(grid), dim3(WM * WN * 64),
                          0, s, nullptr, done, 0, x, Wp, cf, cb, M, N, K, k_len, plane_stride,
                          tiles_m, tiles_n, split);
    return check_launch("gemm_bf16_kernel");
  }
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, NB, WM, WN>), dim3(grid), dim3(WM * WN * 64), 0, s,
                     x, Wp, cf, cb, M, N, K, k_len, plane_stride, tiles_m, tiles_n, split);
  return record_after(check_launch("gemm_bf16_kernel"), done, s);
}

template <int BM, int BN, int WM, int WN>
int launch_gemm_nb(const uint16_t* x, const uint16_t* Wp, void* C, bool bf16_out, int M, int N,
                   int K, int split, int stages, long long plane_stride, hipStream_t s,
                   hipEvent_t done, hipEvent_t t0, hipEvent_t t1) {
  // Ring depth.  The 256x256 tile's loads stall on latency with 4 stages, so it takes the
  // deepest ring that fits (5 x 32 KiB).  The smaller tiles run as fast with 4 stages as with
  // deeper rings, and at 4 stages (64 KiB) two 128x128 workgroups fit on one CU, which lets
  // the projections of consecutive chunks share the CUs.  Tests and tuning may ask for
  // another instantiated depth.
  constexpr int STAGE = (BM + BN) * kBK * 2;
  constexpr int DEEP = (160 * 1024) / STAGE > 8 ? 8 : (160 * 1024) / STAGE;
  constexpr int MID = (DEEP + 4) / 2;
  if (stages == 0) stages = (BM == 256 && BN == 256) ? DEEP : 4;
  if (stages == DEEP)
    return launch_gemm_t<BM, BN, DEEP, WM, WN>(x, Wp, C, bf16_out, M, N, K, split, plane_stride, s, done, t0, t1);
  if (stages == 4)
    return launch_gemm_t<BM, BN, 4, WM, WN>(x, Wp, C, bf16_out, M, N, K, split, plane_stride, s, done, t0, t1);
  if (stages == MID)
    return launch_gemm_t<BM, BN, MID, WM, WN>(x, Wp, C, bf16_out, M, N, K, split, plane_stride, s, done, t0, t1);
  return fail(PR_ERR_INVALID_ARG, "projection tile %dx%d has no %d-stage variant (4, %d, %d)", BM,
              BN, stages, MID, DEEP);
}

// Workgroups of one instantiation that the device holds at once (cooperative-launch limit).
template <typename Kern>
int resident_workgroups(Kern kern, int threads, int* out) {
  int dev = 0, per_cu = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                     threads, 0);
  if (e != hipSuccess) return fail(PR_ERR_HIP, "occupancy query: %s", hipGetErrorString(e));
  *out = per_cu * cus;
  return PR_OK;
}

// Scales of the FP8 form (unused otherwise): per-group activation scales read at
// (scale_row0 + row) / scale_rows, and the weight's scale.
struct Fp8Scales {
  const float* x_scales = nullptr;
  int scale_rows = 1;
  int scale_row0 = 0;
  const float* w_scale = nullptr;
};

template <int BM, int BN, int NB, int WM, int WN, int KG, bool FP8 = false, bool SILU = false>
int launch_single_t(const uint16_t* x, const uint16_t* Wp, float* r, const float* w,
                    uint16_t* out, const SingleWs& ws, int M, int N, int K, float eps, int gemma,
                    hipStream_t s, hipEvent_t t0, hipEvent_t t1,
                    const Fp8Scales& sc = Fp8Scales()) {
  auto kern = gemm_add_rmsnorm_kernel<BM, BN, NB, WM, WN, KG, FP8, SILU>;
  constexpr int threads = WM * WN * KG * 64;
  static int resident = 0;  // per instantiation; the library runs on one kind of device
  if (resident == 0) PR_TRY_K(resident_workgroups(kern, threads, &resident));
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = N / BN;
  const int rows_per_round = resident / tiles_n < tiles_m ? resident / tiles_n : tiles_m;
  if (rows_per_round < 1)
    return fail(PR_ERR_UNSUPPORTED, "single launch: %d tiles per row exceed the %d resident "
                "workgroups", tiles_n, resident);
  const unsigned grid = (unsigned)(rows_per_round * tiles_n);
  if (t0 != nullptr) {
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, s, t0, t1, 0, x, Wp, r, w, out,
                          ws.slots, ws.sync, M, N, K, tiles_m, tiles_n, rows_per_round, eps,
                          gemma, ws.fault_mask, ws.spin_limit, ws.pwords, ws.slot_words,
                          ws.pword_words, ws.host_flag, sc.x_scales, sc.scale_rows,
                          sc.scale_row0, sc.w_scale);
  } else {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, s, x, Wp, r, w, out, ws.slots,
                       ws.sync, M, N, K, tiles_m, tiles_n, rows_per_round, eps, gemma,
                       ws.fault_mask, ws.spin_limit, ws.pwords, ws.slot_words, ws.pword_words,
                       ws.host_flag, sc.x_scales, sc.scale_rows, sc.scale_row0, sc.w_scale);
  }
  return check_launch("gemm_add_rmsnorm_kernel");
}

// Pair form (256 x 256 tiles, 8 waves, K split over two workgroups).  Rounds cover whole tile
// rows; every pair and row block of a round is resident at once.
int launch_pair(const uint16_t* x, const uint16_t* Wp, float* r, const float* w, uint16_t* out,
                const SingleWs& ws, int M, int N, int K, float eps, int gemma, hipStream_t s,
                hipEvent_t t0, hipEvent_t t1) {
  auto kern = gemm_add_rmsnorm_pair_kernel<5>;
  constexpr int threads = 512;
  static int resident = 0;
  if (resident == 0) PR_TRY_K(resident_workgroups(kern, threads, &resident));
  const int tiles_m = (M + 255) / 256;
  const int tiles_n = N / 256;
  const int rows_per_round =
      resident / (2 * tiles_n) < tiles_m ? resident / (2 * tiles_n) : tiles_m;
  if (rows_per_round < 1)
    return fail(PR_ERR_UNSUPPORTED, "single launch (pairs): %d workgroups per tile row exceed "
                "the %d resident workgroups", 2 * tiles_n, resident);
  const unsigned grid = (unsigned)(2 * rows_per_round * tiles_n);
  const size_t parities = rows_per_round < tiles_m ? 2 : 1;
  if (ws.xbuf == nullptr || ws.pwords == nullptr || parities * grid * 16384u > ws.xbuf_words)
    return fail(PR_ERR_INVALID_ARG, "single launch (pairs): exchange buffer of %zu words is "
                "smaller than %zu", ws.xbuf_words, parities * grid * 16384u);
  if (t0 != nullptr) {
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, s, t0, t1, 0, x, Wp, r, w, out,
                          ws.slots, ws.sync, ws.pwords, ws.xbuf, M, N, K, tiles_m, tiles_n,
                          rows_per_round, eps, gemma, ws.fault_mask, ws.spin_limit,
                          ws.slot_words, ws.pword_words, ws.host_flag);
  } else {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, s, x, Wp, r, w, out, ws.slots,
                       ws.sync, ws.pwords, ws.xbuf, M, N, K, tiles_m, tiles_n, rows_per_round,
                       eps, gemma, ws.fault_mask, ws.spin_limit, ws.slot_words, ws.pword_words,
                       ws.host_flag);
  }
  return check_launch("gemm_add_rmsnorm_pair_kernel");
}

template <int NV, int WPR, bool YB>
int launch_addnorm_t(const void* y, int y_bf16, int nplanes, long long plane_stride, int round_y,
                     float* r, const float* w, uint16_t* out, int rows, int H, float eps,
                     int gemma, int max_wgs, hipStream_t s, hipEvent_t done, hipEvent_t t0,
                     hipEvent_t t1) {
  constexpr int RPB = WPR <= 4 ? 4 / WPR : 1;
  int groups = (rows + RPB - 1) / RPB;
  if (max_wgs > 0 && groups > max_wgs) groups = max_wgs;
  const unsigned grid = (unsigned)groups;
  if (t0 != nullptr || (done != nullptr && ext_launch_events())) {
    hipExtLaunchKernelGGL((add_rmsnorm_kernel<NV, WPR, YB>), dim3(grid), dim3(64 * WPR * RPB), 0, s,
                          t0, t0 != nullptr ? t1 : done, 0,
                          y_bf16 ? nullptr : static_cast<const float*>(y),
                          y_bf16 ? static_cast<const uint16_t*>(y) : nullptr, nplanes,
                          plane_stride, round_y, r, w, out, rows, H, eps, gemma);
    return t0 != nullptr ? record_after(check_launch("add_rmsnorm_kernel"), done, s)
                         : check_launch("add_rmsnorm_kernel");
  }
  hipLaunchKernelGGL((add_rmsnorm_kernel<NV, WPR, YB>), dim3(grid), dim3(64 * WPR * RPB), 0, s,
                     y_bf16 ? nullptr : static_cast<const float*>(y),
                     y_bf16 ? static_cast<const uint16_t*>(y) : nullptr, nplanes, plane_stride,
                     round_y, r, w, out, rows, H, eps, gemma);
  return record_after(check_launch("add_rmsnorm_kernel"), done, s);
}

}  // namespace

int launch_gemm(const uint16_t* x, const uint16_t* Wp, void* C, bool bf16_out, int M, int N,
                int K, const GemmCfg& cfg, long long plane_stride, void* stream, void* done_event,
                void* start_timing, void* stop_timing) {
  hipEvent_t done = static_cast<hipEvent_t>(done_event);
  hipEvent_t t0 = static_cast<hipEvent_t>(start_timing);
  hipEvent_t t1 = static_cast<hipEvent_t>(stop_timing);
  if (M <= 0) return PR_OK;
  if (K % (2 * kBK * cfg.split) != 0 || N % 64 != 0 || (bf16_out && cfg.split != 1) ||
      cfg.kgroups != 1)
    return fail(PR_ERR_SHAPE, "projection shape M=%d N=%d K=%d split=%d not supported", M, N, K,
                cfg.split);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool eight = cfg.waves == 8;
  if (cfg.bm == 256 && cfg.bn == 256)
    return eight ? launch_gemm_nb<256, 256, 2, 4>(x, Wp, C, bf16_out, M, N, K, cfg.split, cfg.stages, plane_stride, s, done, t0, t1)
                 : launch_gemm_nb<256, 256, 2, 2>(x, Wp, C, bf16_out, M, N, K, cfg.split, cfg.stages, plane_stride, s, done, t0, t1);
  if (cfg.bm == 256 && cfg.bn == 128)
    return eight ? launch_gemm_nb<256, 128, 4, 2>(x, Wp, C, bf16_out, M, N, K, cfg.split, cfg.stages, plane_stride, s, done, t0, t1)
                 : launch_gemm_nb<256, 128, 2, 2>(x, Wp, C, bf16_out, M, N, K, cfg.split, cfg.stages, plane_stride, s, done, t0, t1);
  if (cfg.bm == 128 && cfg.bn == 128)
    return eight ? launch_gemm_nb<128, 128, 2, 4>(x, Wp, C, bf16_out, M, N, K, cfg.split, cfg.stages, plane_stride, s, done, t0, t1)
                 : launch_gemm_nb<128, 128, 2, 2>(x, Wp, C, bf16_out, M, N, K, cfg.split, cfg.stages, plane_stride, s, done, t0, t1);
  return fail(PR_ERR_INVALID_ARG, "no projection tile %dx%d", cfg.bm, cfg.bn);
}

int launch_gemm_add_rmsnorm(const uint16_t* x, const uint16_t* Wp, float* r, const float* w,
                            uint16_t* out, const SingleWs& ws, int M, int N, int K,
                            const GemmCfg& cfg, float eps, int gemma, void* stream,
                            void* start_timing, void* stop_timing) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t t0 = static_cast<hipEvent_t>(start_timing);
  hipEvent_t t1 = static_cast<hipEvent_t>(stop_timing);
  if (M <= 0) return PR_OK;
  if (cfg.split == 2) {
    if (cfg.bm != 256 || cfg.bn != 256 || cfg.waves != 8 || cfg.kgroups != 1 ||
        K % (2 * kBK) != 0 || K < 256 || N % 256 != 0 || N / 256 > 64)
      return fail(PR_ERR_SHAPE, "single launch (pairs): N=%d K=%d with tile %dx%d, %d waves, %d "
                  "K groups not supported (256x256, 8 waves, N a multiple of 256, K >= 256)", N,
                  K, cfg.bm, cfg.bn, cfg.waves, cfg.kgroups);
    return launch_pair(x, Wp, r, w, out, ws, M, N, K, eps, gemma, s, t0, t1);
  }
  const bool r256x128 = cfg.bm == 256 && cfg.bn == 128;
  const bool r192 = cfg.bm == 192 && cfg.bn == 192;
  if (K % (2 * kBK) != 0 || N % cfg.bn != 0 || N / cfg.bn > 64 || cfg.split != 1 ||
      (cfg.waves != 8 && !(cfg.waves == 4 && r256x128) && !(cfg.waves == 12 && r192)) ||
      (r192 && cfg.waves != 12) ||
      (cfg.kgroups != 1 && !(cfg.kgroups == 2 && cfg.waves == 8 && r256x128)))
    return fail(PR_ERR_SHAPE, "single launch: N=%d K=%d with tile %dx%d split %d, %d waves, %d K "
                "groups not supported", N, K, cfg.bm, cfg.bn, cfg.split, cfg.waves, cfg.kgroups);
  if (cfg.bm == 256 && cfg.bn == 256)
    return launch_single_t<256, 256, 5, 2, 4, 1>(x, Wp, r, w, out, ws, M, N, K, eps, gemma, s,
                                                 t0, t1);
  if (r256x128 && cfg.kgroups == 2)
    return launch_single_t<256, 128, 3, 2, 2, 2>(x, Wp, r, w, out, ws, M, N, K, eps, gemma, s,
                                                 t0, t1);
  if (cfg.bm == 256 && cfg.bn == 128 && cfg.waves == 4)
    return launch_single_t<256, 128, 4, 2, 2, 1>(x, Wp, r, w, out, ws, M, N, K, eps, gemma, s,
                                                 t0, t1);
  if (cfg.bm == 256 && cfg.bn == 128)
    return launch_single_t<256, 128, 4, 4, 2, 1>(x, Wp, r, w, out, ws, M, N, K, eps, gemma, s,
                                                 t0, t1);
  if (cfg.bm == 128 && cfg.bn == 128)
    return launch_single_t<128, 128, 4, 2, 4, 1>(x, Wp, r, w, out, ws, M, N, K, eps, gemma, s,
                                                 t0, t1);
  if (r192)
    return launch_single_t<192, 192, 3, 2, 6, 1>(x, Wp, r, w, out, ws, M, N, K, eps, gemma, s,
                                                 t0, t1);
  return fail(PR_ERR_INVALID_ARG, "single launch: no tile %dx%d", cfg.bm, cfg.bn);
}

int launch_gemm_add_rmsnorm_fp8(const uint8_t* xq, const uint8_t* Wq, float* r, const float* w,
                                uint16_t* out, const SingleWs& ws, int M, int N, int K,
                                const GemmCfg& cfg, const float* x_scales, int scale_rows,
                                int scale_row0, const float* w_scale, float eps, int gemma,
                                void* stream, void* start_timing, void* stop_timing) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t t0 = static_cast<hipEvent_t>(start_timing);
  hipEvent_t t1 = static_cast<hipEvent_t>(stop_timing);
  if (M <= 0) return PR_OK;
  if (K % (2 * kBK) != 0 || N % cfg.bn != 0 || N / cfg.bn > 64 || cfg.split != 1 ||
      cfg.waves != 8 || (cfg.kgroups != 1 && !(cfg.kgroups == 2 && cfg.bm == 256 &&
                                               cfg.bn == 128 && K % (4 * kBK) == 0)))
    return fail(PR_ERR_SHAPE, "FP8 single launch: N=%d K=%d with tile %dx%d split %d, %d waves, "
                "%d K groups not supported (K a multiple of 64, 8 waves, two K groups only on "
                "256x128 with K a multiple of 128)", N, K, cfg.bm, cfg.bn, cfg.split, cfg.waves,
                cfg.kgroups);
  Fp8Scales sc;
  sc.x_scales = x_scales;
  sc.scale_rows = scale_rows;
  sc.scale_row0 = scale_row0;
  sc.w_scale = w_scale;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(xq);  // byte arrays (see the kernel)
  const uint16_t* Wp = reinterpret_cast<const uint16_t*>(Wq);
  if (cfg.bm == 256 && cfg.bn == 256)
    return launch_single_t<256, 256, 5, 2, 4, 1, true>(x, Wp, r, w, out, ws, M, N, K, eps, gemma,
                                                       s, t0, t1, sc);
  if (cfg.bm == 256 && cfg.bn == 128 && cfg.kgroups == 2)
    return launch_single_t<256, 128, 3, 2, 2, 2, true>(x, Wp, r, w, out, ws, M, N, K, eps, gemma,
                                                       s, t0, t1, sc);
  if (cfg.bm == 256 && cfg.bn == 128)
    return launch_single_t<256, 128, 4, 4, 2, 1, true>(x, Wp, r, w, out, ws, M, N, K, eps, gemma,
                                                       s, t0, t1, sc);
  if (cfg.bm == 128 && cfg.bn == 128)
    return launch_single_t<128, 128, 4, 2, 4, 1, true>(x, Wp, r, w, out, ws, M, N, K, eps, gemma,
                                                       s, t0, t1, sc);
  return fail(PR_ERR_INVALID_ARG, "FP8 single launch: no tile %dx%d", cfg.bm, cfg.bn);
}

int launch_gemm_add_rmsnorm_silu(const uint16_t* gate_up, const uint16_t* Wp, float* r,
                                 const float* w, uint16_t* out, const SingleWs& ws, int M, int N,
                                 int K, const GemmCfg& cfg, float eps, int gemma, void* stream,
                                 void* start_timing, void* stop_timing) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t t0 = static_cast<hipEvent_t>(start_timing);
  hipEvent_t t1 = static_cast<hipEvent_t>(stop_timing);
  if (M <= 0) return PR_OK;
  if (K % (2 * kBK) != 0 || N % cfg.bn != 0 || N / cfg.bn > 64 || cfg.split != 1 ||
      cfg.kgroups != 1 || cfg.waves != 8)
    return fail(PR_ERR_SHAPE, "SiluAndMul single launch: N=%d K=%d with tile %dx%d split %d, %d "
                "waves not supported (8 waves, one K group)", N, K, cfg.bm, cfg.bn, cfg.split,
                cfg.waves);
  // Stages of gate, up and weight tiles: 48 KiB (256x256: 3 in the ring), 40 KiB (256x128:
  // 4), 24 KiB (128x128: 4).
  if (cfg.bm == 256 && cfg.bn == 256)
    return launch_single_t<256, 256, 3, 2, 4, 1, false, true>(gate_up, Wp, r, w, out, ws, M, N, K,
                                                              eps, gemma, s, t0, t1);
  if (cfg.bm == 256 && cfg.bn == 128)
    return launch_single_t<256, 128, 4, 4, 2, 1, false, true>(gate_up, Wp, r, w, out, ws, M, N, K,
                                                              eps, gemma, s, t0, t1);
  if (cfg.bm == 128 && cfg.bn == 128)
    return launch_single_t<128, 128, 4, 2, 4, 1, false, true>(gate_up, Wp, r, w, out, ws, M, N, K,
                                                              eps, gemma, s, t0, t1);
  return fail(PR_ERR_INVALID_ARG, "SiluAndMul single launch: no tile %dx%d", cfg.bm, cfg.bn);
}

int launch_add_rmsnorm(const void* y, int y_bf16, int nplanes, long long plane_stride,
                       int round_y, float* r, const float* w, uint16_t* out, int rows, int H,
                       float eps, int gemma, int max_wgs, void* stream, void* done_event,
                       void* start_timing, void* stop_timing) {
  if (rows <= 0) return PR_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t done = static_cast<hipEvent_t>(done_event);
  hipEvent_t t0 = static_cast<hipEvent_t>(start_timing);
  hipEvent_t t1 = static_cast<hipEvent_t>(stop_timing);
  // Waves per row: the fewest that give an instantiated row share of at most 8 float4 per lane
  // (when the segment count allows), then more (within the segment count and instantiated
  // shares) until the launch has >= 2048 waves.  Whether the
  // register-resident kernel is used at all depends on H only, and its result does not depend
  // on the waves per row, so every row count gives the same result for a given H.
  if (H % 256 == 0) {
    // At most 16 float4 per lane: the residual, the running y and one plane batch stay in
    // registers together.
    auto inst = [](int nv) {
      return (nv >= 1 && nv <= 8) || nv == 10 || nv == 12 || nv == 14 || nv == 16;
    };
    const int n4 = H / 256;  // float4 per lane for one wave per row
    const int segs = n4 % 8 == 0 ? 8 : (n4 % 4 == 0 ? 4 : (n4 % 2 == 0 ? 2 : 1));
    // At most 8 float4 per lane where the segments allow it (16 per lane takes the whole
    // register file and leaves one wave per SIMD).
    int wpr = 1;
    while (wpr < segs && (!inst(n4 / wpr) || n4 / wpr > 8)) wpr *= 2;
    while (inst(n4 / wpr) && 2 * wpr <= segs && inst(n4 / (2 * wpr)) &&
           (long long)rows * wpr < 2048)
      wpr *= 2;
    const int nv = n4 / wpr;
#define PR_AN(NV_, W_)                                                                        \
  if (nv == NV_ && wpr == W_ && n4 == NV_ * W_)                                               \
    return y_bf16 ? launch_addnorm_t<NV_, W_, true>(y, y_bf16, nplanes, plane_stride, round_y, r, \
                                                    w, out, rows, H, eps, gemma, max_wgs, s,   \
                                                    done, t0, t1)                              \
                  : launch_addnorm_t<NV_, W_, false>(y, y_bf16, nplanes, plane_stride, round_y,  \
                                                     r, w, out, rows, H, eps, gemma, max_wgs, \
                                                     s, done, t0, t1);
#define PR_AN_ALL(NV_) PR_AN(NV_, 1) PR_AN(NV_, 2) PR_AN(NV_, 4) PR_AN(NV_, 8)
    PR_AN_ALL(1) PR_AN_ALL(2) PR_AN_ALL(3) PR_AN_ALL(4) PR_AN_ALL(5) PR_AN_ALL(6) PR_AN_ALL(7)
    PR_AN_ALL(8) PR_AN_ALL(10) PR_AN_ALL(12) PR_AN_ALL(14) PR_AN_ALL(16)
#undef PR_AN_ALL
#undef PR_AN
  }
  int groups = (rows + 3) / 4;
  if (max_wgs > 0 && groups > max_wgs) groups = max_wgs;
  const unsigned grid = (unsigned)groups;
  if (t0 != nullptr) {
    hipExtLaunchKernelGGL(add_rmsnorm_generic_kernel, dim3(grid), dim3(256), 0, s, t0, t1, 0,
                          y_bf16 ? nullptr : static_cast<const float*>(y),
                          y_bf16 ? static_cast<const uint16_t*>(y) : nullptr, nplanes,
                          plane_stride, round_y, r, w, out, rows, H, eps, gemma);
    return record_after(check_launch("add_rmsnorm_generic_kernel"), done, s);
  }
  hipLaunchKernelGGL(add_rmsnorm_generic_kernel, dim3(grid), dim3(256), 0, s,
                     y_bf16 ? nullptr : static_cast<const float*>(y),
                     y_bf16 ? static_cast<const uint16_t*>(y) : nullptr, nplanes, plane_stride,
                     round_y, r, w, out, rows, H, eps, gemma);
  return record_after(check_launch("add_rmsnorm_generic_kernel"), done, s);
}

int launch_prepare_weight(const uint16_t* src, int src_layout, uint16_t* dst, int K, int H,
                          void* stream) {
  const long long total = (long long)(K / 8) * H;
  if (total == 0) return PR_OK;
  const unsigned grid = (unsigned)((total + 255) / 256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (src_layout == PR_WEIGHT_OUT_IN)
    hipLaunchKernelGGL(prepare_weight_out_in_kernel, dim3(grid), dim3(256), 0, s, src, dst, K, H);
  else
    hipLaunchKernelGGL(prepare_weight_in_out_kernel, dim3(grid), dim3(256), 0, s, src, dst, K, H);
  return check_launch("prepare_weight");
}

int launch_delay(int iters, void* stream) {
  hipLaunchKernelGGL(delay_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), iters);
  return check_launch("delay_kernel");
}

int launch_fill_nan(float* p, size_t n, void* stream) {
  if (n == 0) return PR_OK;
  hipLaunchKernelGGL(fill_nan_kernel, dim3(1024), dim3(256), 0, static_cast<hipStream_t>(stream),
                     p, n);
  return check_launch("fill_nan_kernel");
}

int launch_fill_bf16_hash(uint16_t* p, size_t n, uint32_t seed, float scale, void* stream) {
  if (n == 0) return PR_OK;
  hipLaunchKernelGGL(fill_bf16_hash_kernel, dim3(2048), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p, n, seed, scale);
  return check_launch("fill_bf16_hash_kernel");
}

int launch_fill_f32_hash(float* p, size_t n, uint32_t seed, float scale, float offset,
                         void* stream) {
  if (n == 0) return PR_OK;
  hipLaunchKernelGGL(fill_f32_hash_kernel, dim3(2048), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p, n, seed, scale, offset);
  return check_launch("fill_f32_hash_kernel");
}

}  // namespace pr

#ifdef PR_PHASE_STAMPS
// Host access to the phase stamps of the diagnostic library (not part of the default
// library's ABI).  pr_phase_stamps_layout gives the workgroups covered and the 64-bit words per
// workgroup; pr_phase_stamps_read copies `words` words of the current device's stamps to host
// memory after synchronising the device; pr_phase_stamps_clear synchronises the device and
// zeroes them.
// Each returns 0 or PR_ERR_HIP.
extern "C" int pr_phase_stamps_layout(int* groups, int* words_per_group) {
  *groups = pr::kStampGroups;
  *words_per_group = pr::kStampWords;
  return PR_OK;
}

extern "C" int pr_phase_stamps_read(unsigned long long* dst, int words) {
  if (words < 0 || words > pr::kStampGroups * pr::kStampWords) return PR_ERR_INVALID_ARG;
  if (hipDeviceSynchronize() != hipSuccess) return PR_ERR_HIP;
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(pr::pr_phase_stamps),
                             (size_t)words * sizeof(unsigned long long)) == hipSuccess
             ? PR_OK
             : PR_ERR_HIP;
}

extern "C" int pr_phase_stamps_clear(void) {
  void* p = nullptr;
  if (hipDeviceSynchronize() != hipSuccess) return PR_ERR_HIP;  // no launch still stamping
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(pr::pr_phase_stamps)) != hipSuccess) return PR_ERR_HIP;
  if (hipMemset(p, 0, sizeof(unsigned long long) * pr::kStampGroups * pr::kStampWords) !=
      hipSuccess)
    return PR_ERR_HIP;
  return hipDeviceSynchronize() == hipSuccess ? PR_OK : PR_ERR_HIP;
}
#endif
