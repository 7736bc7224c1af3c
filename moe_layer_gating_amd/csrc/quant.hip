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

// max |src| over n bf16 values (n a multiple of 8, src 16-byte aligned).
__global__ __launch_bounds__(256) void amax_bf16_kernel(const uint16_t* __restrict__ src, long n8,
                                                        uint32_t* amax_bits) {
  __shared__ float part[4];
  float m = 0.f;
  const i32x4* s4 = reinterpret_cast<const i32x4*>(src);
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n8;
       i += (long)gridDim.x * blockDim.x) {
    i32x4 v = s4[i];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      uint32_t u = (uint32_t)v[q];
      m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(u & 0xffffu))));
      m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(u >> 16))));
    }
  }
  m = wave_max(m);
  if (lane_id() == 0) part[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    atomicMax(amax_bits, __float_as_uint(b));
  }
}

hipError_t launch_amax_bf16(const uint16_t* src, long n, uint32_t* amax_bits, hipStream_t st) {
  long n8 = n / 8;
  long blocks = (n8 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  amax_bf16_kernel<<<(int)blocks, 256, 0, st>>>(src, n8, amax_bits);
  return hipGetLastError();
}

// codes = e4m3(bf16 * 448/amax); 8 values per thread per step.
__global__ __launch_bounds__(256) void quant_e4m3_kernel(const uint16_t* __restrict__ src, long n8,
                                                         const uint32_t* __restrict__ amax_bits,
                                                         uint8_t* __restrict__ dst) {
  const float r = amax_to_mult(*amax_bits);
  const i32x4* s4 = reinterpret_cast<const i32x4*>(src);
  uint2* d2 = reinterpret_cast<uint2*>(dst);
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n8;
       i += (long)gridDim.x * blockDim.x) {
    i32x4 v = s4[i];
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int q = 0; q < 2; q++) {
      uint32_t u = (uint32_t)v[q];
      lo |= f32_to_e4m3(bf16_to_f32((uint16_t)(u & 0xffffu)) * r) << (16 * q);
      lo |= f32_to_e4m3(bf16_to_f32((uint16_t)(u >> 16)) * r) << (16 * q + 8);
    }
#pragma unroll
    for (int q = 0; q < 2; q++) {
      uint32_t u = (uint32_t)v[q + 2];
      hi |= f32_to_e4m3(bf16_to_f32((uint16_t)(u & 0xffffu)) * r) << (16 * q);
      hi |= f32_to_e4m3(bf16_to_f32((uint16_t)(u >> 16)) * r) << (16 * q + 8);
    }
    d2[i] = make_uint2(lo, hi);
  }
}

hipError_t launch_quant_e4m3(const uint16_t* src, long n, const uint32_t* amax_bits, uint8_t* dst,
                             hipStream_t st) {
  long n8 = n / 8;
  long blocks = (n8 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  quant_e4m3_kernel<<<(int)blocks, 256, 0, st>>>(src, n8, amax_bits, dst);
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
