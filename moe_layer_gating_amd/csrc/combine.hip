// combine.hip -- top-k weighted aggregation of the expert outputs.
//
// Expert aggregation is the last stage of the fused pass (codebridge-ai.com,
// "aws-moe-kernel-wgmma-triton-ttft", section "2. Backend routing";
// agentic-affairs.com, "Triton improves the FP8 execution path").
//   out[t][m] = sum_{j<k} w[t][j] * y[inv_perm[t*k+j]][m]
// summed in fp32 in slot order j = 0..k-1 and rounded once; each output row
// is written exactly once, by one thread per 8 consecutive features, in
// blocks of 128 threads (a 7168-feature row is 7 whole blocks; with blocks
// of 256 the fourth block of every row was half idle, and the prefill
// aggregation ran 4% slower).  y is
// fp32, or bf16 (YB: the FP8 fused path of many-token layers: one 16-byte
// load per slot), widened exactly before the sum.
#include "moe_common.h"

namespace moe {

template <int MODE, bool YB>
__global__ __launch_bounds__(128) void combine_kernel(const void* __restrict__ y,
                                                      const int32_t* __restrict__ inv_perm,
                                                      const float* __restrict__ w, int T, int H,
                                                      int k, int blocks_per_row,
                                                      void* __restrict__ out) {
  const int t = blockIdx.x / blocks_per_row;
  const int m = ((blockIdx.x - t * blocks_per_row) * blockDim.x + threadIdx.x) * 8;
  if (t >= T || m >= H) return;
  // every slot's position and weight first, then every slot's y row: two
  // dependent round trips instead of two per slot (k <= 16)
  int p[16];
  float wj[16];
#pragma unroll
  for (int j = 0; j < 16; j++)
    if (j < k) {
      p[j] = inv_perm[(size_t)t * k + j];
      wj[j] = w[(size_t)t * k + j];
    }
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  if constexpr (YB) {
    uint4 u[16];  // raw bf16 rows, widened exactly at the sum
#pragma unroll
    for (int j = 0; j < 16; j++)
      if (j < k)
        u[j] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(y) +
                                               (size_t)p[j] * H + m);
#pragma unroll
    for (int j = 0; j < 16; j++)
      if (j < k) {  // slot order j = 0..k-1
        const f32x4 v0 = {__uint_as_float(u[j].x << 16), __uint_as_float(u[j].x & 0xffff0000u),
                          __uint_as_float(u[j].y << 16), __uint_as_float(u[j].y & 0xffff0000u)};
        const f32x4 v1 = {__uint_as_float(u[j].z << 16), __uint_as_float(u[j].z & 0xffff0000u),
                          __uint_as_float(u[j].w << 16), __uint_as_float(u[j].w & 0xffff0000u)};
        a0 += wj[j] * v0;
        a1 += wj[j] * v1;
      }
  } else {
    f32x4 v0[16], v1[16];
#pragma unroll
    for (int j = 0; j < 16; j++)
      if (j < k) {
        const size_t o = (size_t)p[j] * H + m;
        v0[j] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(y) + o);
        v1[j] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(y) + o + 4);
      }
#pragma unroll
    for (int j = 0; j < 16; j++)
      if (j < k) {  // slot order j = 0..k-1
        a0 += wj[j] * v0[j];
        a1 += wj[j] * v1[j];
      }
  }
  const size_t oo = (size_t)t * H + m;
  if (MODE == MOE_F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + oo) = a0;
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + oo + 4) = a1;
  } else {
    const uint4 r = {(uint32_t)f32_to_bf16(a0[0]) | ((uint32_t)f32_to_bf16(a0[1]) << 16),
                     (uint32_t)f32_to_bf16(a0[2]) | ((uint32_t)f32_to_bf16(a0[3]) << 16),
                     (uint32_t)f32_to_bf16(a1[0]) | ((uint32_t)f32_to_bf16(a1[1]) << 16),
                     (uint32_t)f32_to_bf16(a1[2]) | ((uint32_t)f32_to_bf16(a1[3]) << 16)};
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + oo) = r;
  }
}

hipError_t launch_combine(int mode, const void* y, bool y_bf16, const int32_t* inv_perm,
                          const float* w, int T, int H, int k, void* out, hipStream_t st) {
  const int bpr = (H / 8 + 127) / 128;
  const long grid = (long)bpr * T;
  if (grid <= 0) return hipSuccess;
  if (mode == MOE_F32 && y_bf16) return hipErrorInvalidValue;
  if (mode == MOE_F32)
    combine_kernel<MOE_F32, false><<<grid, 128, 0, st>>>(y, inv_perm, w, T, H, k, bpr, out);
  else if (y_bf16)
    combine_kernel<MOE_BF16, true><<<grid, 128, 0, st>>>(y, inv_perm, w, T, H, k, bpr, out);
  else
    combine_kernel<MOE_BF16, false><<<grid, 128, 0, st>>>(y, inv_perm, w, T, H, k, bpr, out);
  return hipGetLastError();
}

}  // namespace moe
