// SiluAndMul kernel (the step before down_proj) and its launcher.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "pr_internal.h"

namespace pr {
namespace {

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN stays a quiet NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_f32(uint32_t b) { return __uint_as_float(b << 16); }

// --------------------------------------------------------------------------------------------
// SiluAndMul on the merged gate/up projection output ("Plugin Architecture" page, SiluAndMul
// row): row t of gate_up holds gate in columns [0, K) and up in [K, 2K); x[t][c] =
// silu(gate) * up in fp32, silu(g) = g / (1 + e^-g), rounded once to bf16.  Elementwise and
// HBM-bound (6 bytes per element of x).  Workgroups stride over rows and threads over a row's
// 16-byte vectors of 8 columns, U vectors per step with all their loads issued before any use,
// so no index needs a division.  gate and up are read once, with streaming loads, so that
// they do not evict the projection's weight from the Infinity Cache.  x is stored at device
// scope (sc1 buffer stores), so its lines go through the L2 to memory as they are written
// instead of staying dirty until the launch's end.  The exponential is the device's native one (__expf, a
// scaled v_exp_f32: relative error near 1e-6, far below the half ulp of the bf16 result) and
// the quotient an ordinary IEEE division.  Zero columns of the load-time padding give zeros.
// --------------------------------------------------------------------------------------------
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
constexpr int kSiluThreads = 256;  // threads per workgroup; the column loop strides by it

template <int U>
__global__ void __launch_bounds__(kSiluThreads) silu_mul_kernel(const uint16_t* __restrict__ gu,
                                                                uint16_t* __restrict__ x, int T,
                                                                int K) {
  const int kvec = K / 8;
  for (int t = blockIdx.x; t < T; t += gridDim.x) {
    const uint4* grow = reinterpret_cast<const uint4*>(gu + (long long)t * 2 * K);
    const uint4* urow = grow + kvec;
    // Word 3 of a gfx9 buffer resource for raw accesses (data format 32 bits: range-checked).
    const __amdgpu_buffer_rsrc_t rs_x =
        __builtin_amdgcn_make_buffer_rsrc(x + (long long)t * K, 0, K * 2, 0x00020000);
    for (int c0 = threadIdx.x; c0 < kvec; c0 += kSiluThreads * U) {
      uint4 g[U], u[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int c = c0 + kSiluThreads * i;
        if (c < kvec) {
          const v4u gv = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(grow) + c);
          const v4u uv = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(urow) + c);
          g[i] = make_uint4(gv.x, gv.y, gv.z, gv.w);
          u[i] = make_uint4(uv.x, uv.y, uv.z, uv.w);
        }
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int c = c0 + kSiluThreads * i;
        if (c < kvec) {
          const uint32_t gw[4] = {g[i].x, g[i].y, g[i].z, g[i].w};
          const uint32_t uw[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
          uint32_t o[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float g0 = bf16_f32(gw[j] & 0xffffu), g1 = bf16_f32(gw[j] >> 16);
            const float u0 = bf16_f32(uw[j] & 0xffffu), u1 = bf16_f32(uw[j] >> 16);
            const float x0 = g0 / (1.0f + __expf(-g0)) * u0;
            const float x1 = g1 / (1.0f + __expf(-g1)) * u1;
            o[j] = bf16_rne(x0) | (bf16_rne(x1) << 16);
          }
          __builtin_amdgcn_raw_buffer_store_b128(v4u{o[0], o[1], o[2], o[3]}, rs_x, c * 16, 0,
                                                 16 /* sc1 */);
        }
      }
    }
  }
}

}  // namespace

int launch_silu_mul(const uint16_t* gate_up, uint16_t* x, int T, int K, void* stream) {
  if (T <= 0) return PR_OK;
  constexpr int kU = 4;
  // One row per workgroup up to 16 workgroups per CU; longer inputs stride over rows.
  const int grid = std::min(T, 16 * kNumCUs);
  hipLaunchKernelGGL(silu_mul_kernel<kU>, dim3(grid), dim3(kSiluThreads), 0,
                     static_cast<hipStream_t>(stream), gate_up, x, T, K);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PR_ERR_HIP, "silu_mul_kernel: %s", hipGetErrorString(e));
  return PR_OK;
}


}  // namespace pr
