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

// Nearest E4M3 code of v (ties to the even code), magnitudes at or above 448 clamped to 448,
// the sign kept (-0 -> 0x80), NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(v);
  if (!(a == a)) return 0x7Fu;
  if (a >= kE4M3Max) return sign | 0x7Eu;
  // Below 2^-6 the codes are the subnormals m * 2^-9 (m = 8 is the smallest normal, code 8):
  // a * 512 is exact and rintf rounds half to even.
  if (a < 0.015625f) return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  // Normal: keep 3 of fp32's 23 mantissa bits, rounding to nearest even (a carry moves into
  // the exponent), and rebias the exponent from 127 to 7.
  const uint32_t au = u & 0x7FFFFFFFu;
  const uint32_t r = au + 0x7FFFFu + ((au >> 20) & 1u);
  const uint32_t code = (r >> 20) - (120u << 3);
  return sign | min(code, 0x7Eu);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Largest |value| of each row: one wave per row, 16-byte loads of 8 bf16 values; bf16
// magnitudes order like their bit patterns with the sign cleared, so an integer max is exact.
__global__ void __launch_bounds__(256)
    fp8_row_amax_kernel(const uint16_t* __restrict__ src, float* __restrict__ row_amax, int rows,
                        int cols) {
  const int lane = threadIdx.x & 63;
  const int nvec = cols / 8;
  for (int row = blockIdx.x * 4 + (int)(threadIdx.x >> 6); row < rows; row += gridDim.x * 4) {
    const uint4* p = reinterpret_cast<const uint4*>(src + (long long)row * cols);
    uint32_t m = 0;
    for (int c = lane; c < nvec; c += 64) {
      const uint4 v = p[c];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
    }
    m = wave_max_u32(m);
    if (lane == 0) row_amax[row] = bf16_value(m);
  }
}

// Codes of each row with its group's scale: one wave per row.  The wave takes the group's
// largest magnitude from the row maxima, forms the scale and converts its row, 8 values per
// lane and step; the first row of a group also stores the group's scale.
__global__ void __launch_bounds__(256)
    fp8_quantize_kernel(const uint16_t* __restrict__ src, const float* __restrict__ row_amax,
                        uint8_t* __restrict__ dst, float* __restrict__ scales, int rows,
                        int cols, int group_rows) {
  const int lane = threadIdx.x & 63;
  const int nvec = cols / 8;
  for (int row = blockIdx.x * 4 + (int)(threadIdx.x >> 6); row < rows; row += gridDim.x * 4) {
    const int g = row / group_rows;
    const int r0 = g * group_rows, r1 = min(rows, r0 + group_rows);
    float amax = 0.0f;
    for (int r = r0 + lane; r < r1; r += 64) amax = fmaxf(amax, row_amax[r]);
    amax = wave_max_f32(amax);
    const float scale = amax == 0.0f ? 1.0f : amax / kE4M3Max;
    if (row == r0 && lane == 0) scales[g] = scale;
    const uint4* p = reinterpret_cast<const uint4*>(src + (long long)row * cols);
    uint2* q = reinterpret_cast<uint2*>(dst + (long long)row * cols);
    for (int c = lane; c < nvec; c += 64) {
      const uint4 v = p[c];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t b[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b[2 * j] = e4m3_code(bf16_value(w[j] & 0xFFFFu) / scale);
        b[2 * j + 1] = e4m3_code(bf16_value(w[j] >> 16) / scale);
      }
      q[c] = make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                        b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
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

int launch_quantize_fp8(const uint16_t* src, uint8_t* dst, float* scales, float* row_amax,
                        int rows, int cols, int group_rows, void* stream) {
  if (rows <= 0) return PR_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned grid = (unsigned)std::min((rows + 3) / 4, 16 * kNumCUs);
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
