// quant.hip -- dynamic per-tensor FP8 (OCP e4m3fn) quantisation of the
// activations entering the expert GEMMs.
//
// FP8 tensor scaling is one of the steps the fused FP8 pass folds together
// with the matrix products (agentic-affairs.com, "Triton improves the FP8
// execution path"; codebridge-ai.com, "aws-moe-kernel-wgmma-triton-ttft",
// section "2. Backend routing").  The scale of a tensor a is
// s = fl32(amax(a) / 448), the codes are e4m3(fl32(a * fl32(448 / amax)))
// rounded to nearest even and saturated to +-448; amax = 0 gives s = 1 and
// multiplier 1.  amax is collected with integer atomics on the fp32 bit
// pattern, which order like the values for non-negative floats, so the
// result does not depend on scheduling.
#include "moe_common.h"

namespace moe {

__device__ __forceinline__ float amax_to_mult(uint32_t bits) {
  float a = __uint_as_float(bits);
  return a > 0.f ? 448.0f / a : 1.0f;
}

__device__ __forceinline__ float amax_to_scale(uint32_t bits) {
  float a = __uint_as_float(bits);
  return a > 0.f ? a / 448.0f : 1.0f;
}

// max |src| over n bf16 values (n a multiple of 8, src 16-byte aligned); each
// thread keeps four 16-byte loads in flight.  Blocks of 1024 threads and at
// most 512 of them: every block ends with one access to the single amax
// word, and those same-address accesses serialise (a probe on a 59 MB tensor:
// 2048 blocks of 256 threads took 46 us, the same reads without the atomics
// 28 us).
__global__ __launch_bounds__(1024) void amax_bf16_kernel(const uint16_t* __restrict__ src, long n8,
                                                         uint32_t* amax_bits) {
  __shared__ float part[16];
  float m = 0.f;
  const i32x4* s4 = reinterpret_cast<const i32x4*>(src);
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i0 = blockIdx.x * (long)blockDim.x + threadIdx.x; i0 < n8; i0 += 4 * stride) {
    i32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const long i = i0 + u * stride;
      v[u] = i < n8 ? s4[i] : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 4; u++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        uint32_t w = (uint32_t)v[u][q];
        m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(w & 0xffffu))));
        m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(w >> 16))));
      }
  }
  m = wave_max(m);
  if (lane_id() == 0) part[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    // read first: most blocks then skip the atomic on the single address
    float mb = part[0];
#pragma unroll
    for (int i = 1; i < 16; i++) mb = fmaxf(mb, part[i]);
    const uint32_t b = __float_as_uint(mb);
    if (b > __atomic_load_n(amax_bits, __ATOMIC_RELAXED)) atomicMax(amax_bits, b);
  }
}

hipError_t launch_amax_bf16(const uint16_t* src, long n, uint32_t* amax_bits, hipStream_t st) {
  long n8 = n / 8;
  long blocks = (n8 + 1023) / 1024;  // small tensors still spread over every CU
  if (blocks > 512) blocks = 512;
  if (blocks < 1) blocks = 1;
  amax_bf16_kernel<<<(int)blocks, 1024, 0, st>>>(src, n8, amax_bits);
  return hipGetLastError();
}

// codes = e4m3(bf16 * 448/amax); 8 values per 16-byte load, four loads in
// flight per thread.
__global__ __launch_bounds__(256) void quant_e4m3_kernel(const uint16_t* __restrict__ src, long n8,
                                                         const uint32_t* __restrict__ amax_bits,
                                                         uint8_t* __restrict__ dst) {
  const float r = amax_to_mult(*amax_bits);
  const i32x4* s4 = reinterpret_cast<const i32x4*>(src);
  uint2* d2 = reinterpret_cast<uint2*>(dst);
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i0 = blockIdx.x * (long)blockDim.x + threadIdx.x; i0 < n8; i0 += 4 * stride) {
    i32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const long i = i0 + u * stride;
      v[u] = i < n8 ? s4[i] : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const long i = i0 + u * stride;
      if (i < n8) d2[i] = bf16x8_to_e4m3x8(v[u], r);
    }
  }
}

hipError_t launch_quant_e4m3(const uint16_t* src, long n, const uint32_t* amax_bits, uint8_t* dst,
                             hipStream_t st) {
  long n8 = n / 8;
  long blocks = (n8 + 1023) / 1024;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  quant_e4m3_kernel<<<(int)blocks, 256, 0, st>>>(src, n8, amax_bits, dst);
  return hipGetLastError();
}

// scales = {amax / 448 (1 if amax = 0), amax}, from amax bits held in
// scales[1] by the amax pass
__global__ void finish_scale_kernel(float* scales) {
  if (threadIdx.x == 0) {
    const uint32_t b = __float_as_uint(scales[1]);
    scales[0] = amax_to_scale(b);
  }
}

hipError_t launch_finish_scale(float* scales, hipStream_t st) {
  finish_scale_kernel<<<1, 64, 0, st>>>(scales);
  return hipGetLastError();
}

// act_scales = {s_x, s_h, amax_x, amax_h}
__global__ void write_scales_kernel(const Ctrl* ctrl, float* act_scales) {
  if (threadIdx.x == 0) {
    act_scales[0] = amax_to_scale(ctrl->amax_x_bits);
    act_scales[1] = amax_to_scale(ctrl->amax_h_bits);
    act_scales[2] = __uint_as_float(ctrl->amax_x_bits);
    act_scales[3] = __uint_as_float(ctrl->amax_h_bits);
  }
}

hipError_t launch_write_scales(const Ctrl* ctrl, float* act_scales, hipStream_t st) {
  write_scales_kernel<<<1, 64, 0, st>>>(ctrl, act_scales);
  return hipGetLastError();
}

}  // namespace moe
