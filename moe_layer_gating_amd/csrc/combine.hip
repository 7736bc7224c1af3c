// combine.hip -- top-k weighted aggregation of the expert outputs.
//
// Expert aggregation is the last stage of the fused pass (codebridge-ai.com,
// "aws-moe-kernel-wgmma-triton-ttft", section "2. Backend routing";
// agentic-affairs.com, "Triton improves the FP8 execution path").
//   out[t][m] = sum_{j<k} w[t][j] * y[inv_perm[t*k+j]][m]
// summed in fp32 in slot order j = 0..k-1 and rounded once; each output row
// is written exactly once, by one thread per 4 consecutive features.
#include "moe_common.h"

namespace moe {

template <int MODE>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ inv_perm,
                                                      const float* __restrict__ w, int T, int H,
                                                      int k, int blocks_per_row,
                                                      void* __restrict__ out) {
  const int t = blockIdx.x / blocks_per_row;
  const int m = ((blockIdx.x - t * blocks_per_row) * blockDim.x + threadIdx.x) * 4;
  if (t >= T || m >= H) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; j++) {
    const float wj = w[(size_t)t * k + j];
    const int p = inv_perm[(size_t)t * k + j];
    f32x4 v = *reinterpret_cast<const f32x4*>(y + (size_t)p * H + m);
    acc += wj * v;
  }
  if (MODE == MOE_F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + (size_t)t * H + m) = acc;
  } else {
    uint32_t lo = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
    uint32_t hi = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + (size_t)t * H + m) =
        make_uint2(lo, hi);
  }
}

hipError_t launch_combine(int mode, const float* y, const int32_t* inv_perm, const float* w, int T,
                          int H, int k, void* out, hipStream_t st) {
  const int bpr = (H / 4 + 255) / 256;
  const long grid = (long)bpr * T;
  if (grid <= 0) return hipSuccess;
  if (mode == MOE_F32)
    combine_kernel<MOE_F32><<<grid, 256, 0, st>>>(y, inv_perm, w, T, H, k, bpr, out);
  else
    combine_kernel<MOE_BF16><<<grid, 256, 0, st>>>(y, inv_perm, w, T, H, k, bpr, out);
  return hipGetLastError();
}

}  // namespace moe
