// FP8 (OCP E4M3) inputs of the quantised projection ("TPSP Design" page, section 5 To-do:
// quantized projections with their scales handled across microchunks): scaled quantisation of
// bf16 activations or weights by groups of rows, and the weight's matrix-core layout.
//
// E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; no infinities; S.1111.111 is NaN;
// the largest finite magnitude is 448.  A group's scale is its largest magnitude / 448 (1 for
// an all-zero group) and a code is value / scale in fp32 (an IEEE division), rounded to the
// nearest E4M3 value with ties to even and clamped to +-448.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "pr_internal.h"

namespace pr {
namespace {

constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float bf16_value(uint32_t b) { return __uint_as_float(b << 16); }

// E4M3 code conversion: v_cvt_pk_fp8_f32, gfx950's OCP E4M3 conversion, rounds to the
// nearest value with ties to even and keeps the sign (-0 -> 0x80); inputs are clamped to +-448
// first.  HI selects the word the two codes go to (first value in the lower byte).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b, uint32_t old) {
  const float ca = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
  const float cb = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, (int)old, HI);
}

// Codes of 8 bf16 values (one 16-byte vector) divided by scale: the quotient is an IEEE fp32
// division, and a NaN quotient gives 0x7F.
__device__ __forceinline__ uint2 e4m3_codes8(const uint4& v, float scale) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float q[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    q[2 * j] = bf16_value(w[j] & 0xFFFFu) / scale;
    q[2 * j + 1] = bf16_value(w[j] >> 16) / scale;
  }
  uint32_t p[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    p[h] = e4m3_pair<true>(q[4 * h + 2], q[4 * h + 3],
                           e4m3_pair<false>(q[4 * h], q[4 * h + 1], 0u));
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (q[4 * h + e] != q[4 * h + e]) p[h] = (p[h] & ~(0xFFu << (8 * e))) | (0x7Fu << (8 * e));
  }
  return make_uint2(p[0], p[1]);
}

// 16-byte vectors a lane loads before it uses any of them: a row of 4096 bf16 values is one
// batch, so every load of a wave is in flight at once.
constexpr int kQuantU = 8;

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Loads of one batch: kQuantU 16-byte vectors per lane, vector c0 + 64 i of the row.  Indexes
// past the row load its last vector again (unconditional loads keep the batch free of
// branches, so the loads stay in flight together): a repeated value does not change a maximum,
// and codes past the row are not stored.
__device__ __forceinline__ void load_batch(const uint4* __restrict__ p, int c0, int nvec,
                                           uint4 (&v)[kQuantU]) {
#pragma unroll
  for (int i = 0; i < kQuantU; ++i) v[i] = p[min(c0 + 64 * i, nvec - 1)];
}

// Largest |value| of each row: one wave per row, 16-byte loads of 8 bf16 values in batches of
// kQuantU per lane; bf16 magnitudes order like their bit patterns with the sign cleared, so an
// integer max is exact.
__global__ void __launch_bounds__(256)
    fp8_row_amax_kernel(const uint16_t* __restrict__ src, float* __restrict__ row_amax, int rows,
                        int cols) {
  const int lane = threadIdx.x & 63;
  const int nvec = cols / 8;
  for (int row = blockIdx.x * 4 + (int)(threadIdx.x >> 6); row < rows; row += gridDim.x * 4) {
    const uint4* p = reinterpret_cast<const uint4*>(src + (long long)row * cols);
    uint32_t m = 0;
    for (int c0 = lane; c0 < nvec; c0 += 64 * kQuantU) {
      uint4 v[kQuantU];
      load_batch(p, c0, nvec, v);
#pragma unroll
      for (int i = 0; i < kQuantU; ++i) {
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
      }
    }
    m = wave_max_u32(m);
    if (lane == 0) row_amax[row] = bf16_value(m);
  }
}

// Codes of each row with its group's scale: one wave per row.  The wave issues the loads of
// its group's row maxima (up to 256 rows at once) and of its first batch, forms the scale from
// the maxima while the batch is in flight, then converts its row in batches of kQuantU 16-byte
// vectors per lane (the waves sharing a SIMD overlap one another's loads and conversions);
// the first row of a group also stores the group's scale.
__global__ void __launch_bounds__(256)
    fp8_quantize_kernel(const uint16_t* __restrict__ src, const float* __restrict__ row_amax,
                        uint8_t* __restrict__ dst, float* __restrict__ scales, int rows,
                        int cols, int group_rows) {
  const int lane = threadIdx.x & 63;
  const int nvec = cols / 8;
  for (int row = blockIdx.x * 4 + (int)(threadIdx.x >> 6); row < rows; row += gridDim.x * 4) {
    const uint4* p = reinterpret_cast<const uint4*>(src + (long long)row * cols);
    uint2* q = reinterpret_cast<uint2*>(dst + (long long)row * cols);
    const int g = row / group_rows;
    const int r0 = g * group_rows, r1 = min(rows, r0 + group_rows);
    // The row maxima are non-negative or NaN, so an integer max of their bits is their max
    // with NaN (above infinity) propagated: a group holding a NaN gets a NaN scale.
    // Indexes past the group read its last row again, which leaves the maximum unchanged.
    uint32_t ra[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ra[j] = __float_as_uint(row_amax[min(r0 + lane + 64 * j, r1 - 1)]);
    uint4 v[kQuantU];
    load_batch(p, lane, nvec, v);
    uint32_t abits = max(max(ra[0], ra[1]), max(ra[2], ra[3]));
    if (r1 - r0 > 256) {  // uniform: groups of more than 256 rows (a per-tensor weight scale)
      for (int r = r0 + 256 + lane; r < r1; r += 64)
        abits = max(abits, __float_as_uint(row_amax[r]));
    }
    const float amax = __uint_as_float(wave_max_u32(abits));
    const float scale = amax == 0.0f ? 1.0f : amax / kE4M3Max;
    if (row == r0 && lane == 0) scales[g] = scale;
    for (int c0 = lane; c0 < nvec; c0 += 64 * kQuantU) {
      if (c0 != lane) load_batch(p, c0, nvec, v);  // the first batch is in flight already
#pragma unroll
      for (int i = 0; i < kQuantU; ++i) {
        const int c = c0 + 64 * i;
        const uint2 code = e4m3_codes8(v[i], scale);
        if (c < nvec) q[c] = code;
      }
    }
  }
}

// One pass for groups of 1, 2 or 4 rows whose rows fit in registers (NV 16-byte vectors per
// lane): a workgroup's four waves take four consecutive rows, so a group never straddles two
// workgroups.  Each wave loads its whole row, takes its largest magnitude (the integer max of
// the magnitude bits, as fp8_row_amax_kernel), the waves of a group combine theirs through LDS,
// and the codes are formed from the registers with the group's scale: the same values and
// arithmetic as the two kernels above, with one read of the row and no workspace.
template <int NV>
__global__ void __launch_bounds__(256)
    fp8_quantize_rows_kernel(const uint16_t* __restrict__ src, uint8_t* __restrict__ dst,
                             float* __restrict__ scales, int rows, int cols, int group_rows) {
  __shared__ uint32_t s_max[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nvec = cols / 8;
  for (int row0 = blockIdx.x * 4; row0 < rows; row0 += gridDim.x * 4) {  // uniform per workgroup
    const int row = row0 + wave;
    // A wave past the last row reads that row again and stores nothing.
    const uint4* p = reinterpret_cast<const uint4*>(src + (long long)min(row, rows - 1) * cols);
    uint4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = p[min(lane + 64 * i, nvec - 1)];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
    }
    m = wave_max_u32(m);
    if (group_rows > 1) {  // uniform
      if (lane == 0) s_max[wave] = row < rows ? m : 0u;
      __syncthreads();
      const int first = wave / group_rows * group_rows;
      uint32_t gm = 0;
      for (int q = 0; q < group_rows; ++q) gm = max(gm, s_max[first + q]);
      m = gm;
      __syncthreads();  // s_max is rewritten by the next rows
    }
    const float amax = bf16_value(m);
    const float scale = amax == 0.0f ? 1.0f : amax / kE4M3Max;
    if (row < rows) {
      if (lane == 0 && row % group_rows == 0) scales[row / group_rows] = scale;
      uint2* q = reinterpret_cast<uint2*>(dst + (long long)row * cols);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c = lane + 64 * i;
        const uint2 code = e4m3_codes8(v[i], scale);
        if (c < nvec) q[c] = code;
      }
    }
  }
}

// dst[((k/16)*H + h)*16 + k%16] = W[h][k]: each output column's 16 consecutive k-values form
// one 16-byte matrix-core operand.  One thread per (k-group, column).
__global__ void prepare_weight_fp8_out_in_kernel(const uint8_t* __restrict__ W,
                                                 uint8_t* __restrict__ dst, int K, int H) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)(K / 16) * H) return;
  const int kg = (int)(idx / H);
  const int h = (int)(idx % H);
  *reinterpret_cast<uint4*>(dst + idx * 16) =
      *reinterpret_cast<const uint4*>(W + (long long)h * K + kg * 16);
}

__global__ void prepare_weight_fp8_in_out_kernel(const uint8_t* __restrict__ Wt,
                                                 uint8_t* __restrict__ dst, int K, int H) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)(K / 16) * H) return;
  const int kg = (int)(idx / H);
  const int h = (int)(idx % H);
  uint32_t p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p[j] = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      p[j] |= (uint32_t)Wt[(long long)(kg * 16 + 4 * j + b) * H + h] << (8 * b);
  }
  *reinterpret_cast<uint4*>(dst + idx * 16) = make_uint4(p[0], p[1], p[2], p[3]);
}

int check(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PR_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return PR_OK;
}

}  // namespace

bool quantize_fp8_single_pass(int cols, int group_rows) {
  // Rows of up to 8192 columns: 16 vectors per lane leave room for three waves per SIMD; with 32
  // (rows of 14336 columns) one wave per SIMD made the pass slower than the two kernels.
  return (group_rows == 1 || group_rows == 2 || group_rows == 4) && cols <= 64 * 8 * 16;
}

int launch_quantize_fp8(const uint16_t* src, uint8_t* dst, float* scales, float* row_amax,
                        int rows, int cols, int group_rows, void* stream) {
  if (rows <= 0) return PR_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned grid = (unsigned)std::min((rows + 3) / 4, 16 * kNumCUs);
  if (quantize_fp8_single_pass(cols, group_rows)) {
    if (cols <= 64 * 8 * 8)
      hipLaunchKernelGGL(fp8_quantize_rows_kernel<8>, dim3(grid), dim3(256), 0, s, src, dst,
                         scales, rows, cols, group_rows);
    else
      hipLaunchKernelGGL(fp8_quantize_rows_kernel<16>, dim3(grid), dim3(256), 0, s, src, dst,
                         scales, rows, cols, group_rows);
    return check("fp8_quantize_rows_kernel");
  }
  hipLaunchKernelGGL(fp8_row_amax_kernel, dim3(grid), dim3(256), 0, s, src, row_amax, rows, cols);
  const int rc = check("fp8_row_amax_kernel");
  if (rc != PR_OK) return rc;
  hipLaunchKernelGGL(fp8_quantize_kernel, dim3(grid), dim3(256), 0, s, src, row_amax, dst, scales,
                     rows, cols, group_rows);
  return check("fp8_quantize_kernel");
}

int launch_prepare_weight_fp8(const uint8_t* src, int src_layout, uint8_t* dst, int K, int H,
                              void* stream) {
  const long long total = (long long)(K / 16) * H;
  if (total == 0) return PR_OK;
  const unsigned grid = (unsigned)((total + 255) / 256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (src_layout == PR_WEIGHT_OUT_IN)
    hipLaunchKernelGGL(prepare_weight_fp8_out_in_kernel, dim3(grid), dim3(256), 0, s, src, dst, K,
                       H);
  else
    hipLaunchKernelGGL(prepare_weight_fp8_in_out_kernel, dim3(grid), dim3(256), 0, s, src, dst, K,
                       H);
  return check("prepare_weight_fp8");
}

}  // namespace pr
