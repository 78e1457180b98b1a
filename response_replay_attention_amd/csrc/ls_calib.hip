// Calibration probes: a measurement aid, not part of the method.
//
// They measure how fast the part sustains bf16 MFMAs under its power limit,
// so that the attention kernels' rate can be set against a ceiling reached on
// the same part rather than only against the published peak (which assumes
// the 2.4 GHz clock).  Every probe keeps two waves per SIMD busy with
// independent accumulation chains for the whole launch and touches global
// memory only to store one float per thread at the end.  The operands are
// random bf16 values (a hash of the thread and step), cycled every MFMA, so
// the matrix datapath toggles as it does on real data.
//
// One step of one wave is 4 x 32768 flop in every mode:
//   mode 0: four v_mfma_f32_32x32x16_bf16, register operands;
//   mode 1: eight v_mfma_f32_16x16x32_bf16, register operands;
//   mode 2: four 32x32x16 MFMAs whose A operands are read from LDS, one
//           16-byte read per lane per MFMA (1 KiB per 32768 flop, the ratio
//           of the attention kernels' K and V^T operand streams);
//   mode 3: eight 16x16x32 MFMAs, each A operand read from LDS serving two
//           MFMAs (the same bytes per flop as mode 2).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ls_internal.hpp"

namespace ls {
namespace {

typedef float f32x4c __attribute__((ext_vector_type(4)));
typedef float f32x16c __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8c __attribute__((ext_vector_type(8)));

constexpr int kCalibThreads = 512;  // eight waves: two per SIMD
constexpr int kCalibLds = 16384;    // bf16 elements (32 KiB) of random data per workgroup

__device__ __forceinline__ float hash_value(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return ((float)(x & 0xffffffU) * (1.0f / 8388608.0f) - 1.0f) * 1.7f;
}

template <int MODE>
__global__ void __launch_bounds__(kCalibThreads, 1) k_calib_mfma(float* out, int iters) {
  __shared__ __attribute__((aligned(16))) __bf16 lds[kCalibLds];
  const unsigned t = blockIdx.x * kCalibThreads + threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (MODE == 2 || MODE == 3) {
    for (int i = threadIdx.x; i < kCalibLds; i += kCalibThreads)
      lds[i] = (__bf16)hash_value(i * 7u + blockIdx.x * 131071u);
    __syncthreads();
  }
  bf16x8c a[8], b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[j][i] = (__bf16)hash_value(t * 131u + j * 17u + i);
      b[j][i] = (__bf16)hash_value(t * 977u + j * 29u + i + 12345u);
    }
  f32x16c c[4];
  f32x4c d[8];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[k][r] = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 4; ++r) d[k][r] = 0.f;
  // LDS modes: each lane reads 16 bytes; a wave reads one contiguous 1 KiB
  // window, which moves with the step (so the reads cannot be hoisted)
  const __bf16* base = lds + lane * 8;
  for (int it = 0; it < iters; it += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (MODE == 0) {
          c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(u + k) & 7], b[(3 * u + k) & 7], c[k], 0, 0, 0);
        } else if (MODE == 1) {
          d[2 * k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[(u + k) & 7], b[(3 * u + k) & 7],
                                                              d[2 * k], 0, 0, 0);
          d[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[(u + k + 4) & 7], b[(3 * u + k + 1) & 7],
                                                                  d[2 * k + 1], 0, 0, 0);
        } else {
          const bf16x8c x = *reinterpret_cast<const bf16x8c*>(base + ((it + 4 * u + k + wave) & 31) * 512);
          if (MODE == 2) {
            c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, b[(3 * u + k) & 7], c[k], 0, 0, 0);
          } else {
            d[2 * k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, b[(3 * u + k) & 7], d[2 * k], 0, 0, 0);
            d[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, b[(3 * u + k + 1) & 7],
                                                                    d[2 * k + 1], 0, 0, 0);
          }
        }
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[k][r];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 4; ++r) s += d[k][r];
  out[t] = s;
}

}  // namespace
}  // namespace ls

extern "C" ls_status ls_calib_mfma(int32_t mode, int32_t workgroups, int32_t iters, float* out,
                                   double* flops, hipStream_t stream) {
  if (mode < 0 || mode > 3 || workgroups < 1 || iters < 8 || iters % 8 != 0 || !out || !flops)
    return LS_ERR_INVALID_ARG;
  *flops = (double)workgroups * (ls::kCalibThreads / 64) * (double)iters * 4.0 * 32768.0;
  const dim3 g(workgroups), b(ls::kCalibThreads);
  switch (mode) {
    case 0: hipLaunchKernelGGL(ls::k_calib_mfma<0>, g, b, 0, stream, out, iters); break;
    case 1: hipLaunchKernelGGL(ls::k_calib_mfma<1>, g, b, 0, stream, out, iters); break;
    case 2: hipLaunchKernelGGL(ls::k_calib_mfma<2>, g, b, 0, stream, out, iters); break;
    default: hipLaunchKernelGGL(ls::k_calib_mfma<3>, g, b, 0, stream, out, iters); break;
  }
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}
