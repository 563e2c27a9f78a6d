// Matrix-core rate probe: the measured counterpart of the published dense
// MFMA peaks that the attention kernels' throughput is quoted against (the
// "% of MFMA peak" of the forward and forward + backward figures).
//
// Every wave runs kChains independent accumulation chains of MFMAs on
// lane-dependent operands, so the matrix pipe always has an independent
// instruction to issue. The first lane of each workgroup records the shader
// cycle counter (s_memtime) and the constant 100 MHz real-time counter
// (s_memrealtime) around its loop: their ratio is the shader clock while the
// pipe is saturated.
#include "device_common.h"
#include "sdpa_internal.h"

namespace sdpa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int kChains = 8;

template <bool FP8>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, uint64_t* stamps) {
  const int lane = threadIdx.x & 63;
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  if constexpr (FP8) {
    i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // Finite e4m3 codes only (0x7f / 0xff are NaN): the low byte stays in
      // 0x38..0x7e for a and 0x30..0x6f for b.
      a[i] = 0x38383838 + lane + i;
      b[i] = 0x30303030 + ((3 * lane + i) & 0x3f);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
    }
  } else {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(1.0f + 0.001f * (lane + i));
      b[i] = (__bf16)(0.5f - 0.001f * (lane - i));
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = Bf16T::mfma(a, b, acc[c]);
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][c];
  // The sum keeps every chain live. It is stored only when it is NaN (never,
  // for these finite operands), by the stamping thread itself after its
  // stamps, where it makes the clock reading obviously wrong.
  if (threadIdx.x == 0) {
    u32x4* out = (u32x4*)(stamps + 4 * blockIdx.x);
    out[0] = u32x4{(uint32_t)t0, (uint32_t)(t0 >> 32), (uint32_t)t1, (uint32_t)(t1 >> 32)};
    out[1] = u32x4{(uint32_t)r0, (uint32_t)(r0 >> 32), (uint32_t)r1, (uint32_t)(r1 >> 32)};
    if (s != s) stamps[4 * blockIdx.x] = 0;
  }
}

}  // namespace

hipError_t launch_mfma_probe(bool fp8, int blocks, int iters, uint64_t* stamps, hipStream_t stream) {
  if (fp8)
    hipLaunchKernelGGL((mfma_probe_kernel<true>), dim3(blocks), dim3(256), 0, stream, iters, stamps);
  else
    hipLaunchKernelGGL((mfma_probe_kernel<false>), dim3(blocks), dim3(256), 0, stream, iters, stamps);
  return hipGetLastError();
}

}  // namespace sdpa
