// router.hip -- the router GEMM in front of the gating: for every token and
// expert, logits[t][e] = x[t] . wg[e] with fp32 accumulation.  x [T,H] and
// wg [E,H] (one row per expert) are in the activation type: fp32 in fp32
// mode, bf16 otherwise (the FP8 mode quantises the experts, not the router).
//
// Token routing is the first stage of the fused operation (readmex.ai, "AWS
// details fused MoE kernel optimizations on SageMaker", summary), and its
// score is what the top-k gating consumes; computing it inside the library
// removes the caller's separate GEMM launch in front of the layer.
//
// Two shapes of work:
//   * few tokens or an expert count that is not a multiple of 128: one block
//     of 8 waves per (expert, group of up to 16 tokens); each wave takes an
//     eighth of the row (fp32 FMAs on 16-byte runs) and adds its 64 partial
//     sums per token, then the 8 wave sums are added in wave order;
//   * otherwise the many-token tiled GEMM of the down projection, with wg as
//     the weight matrix of a single expert (E rows, K = H) and the tokens in
//     tiles of 64: bf16 MFMAs, whose products are exact and whose sums are
//     fp32.
#include "moe_common.h"

namespace moe {

// 16 bytes of an activation row as fp32 values (4 fp32 or 8 bf16).
template <int MODE>
struct Run;
template <>
struct Run<MOE_F32> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const char* p, float* v) {
    const f32x4 r = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = r[i];
  }
};
template <>
struct Run<MOE_BF16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const char* p, float* v) {
    const i32x4 r = *reinterpret_cast<const i32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = __uint_as_float((uint32_t)r[i] << 16);
      v[2 * i + 1] = __uint_as_float((uint32_t)r[i] & 0xffff0000u);
    }
  }
};

constexpr int kRouterTokens = 16;  // tokens per block of the few-token kernel
constexpr int kRouterWaves = 8;    // waves per block, each on 1/8 of the row

// grid (E, ceil(T / 16)), kRouterWaves waves per block.  Wave w takes the
// columns [w H / 8, (w + 1) H / 8); its lane l the 16-byte runs l, l + 64, ...
// of that range (H is a multiple of 128, so H / 8 is a multiple of 16 and
// runs never straddle a range end).  Eight times the waves of one wave per
// (expert, token group): a decode-sized router is latency-bound.
template <int MODE>
__global__ __launch_bounds__(kRouterWaves * 64) void router_small_kernel(
    const char* __restrict__ x, const char* __restrict__ wg, int T, int H, int E,
    float* __restrict__ logits) {
  typedef Run<MODE> R;
  constexpr int ES = 16 / R::N;
  __shared__ float part[kRouterWaves][kRouterTokens];
  const int e = blockIdx.x, t0 = blockIdx.y * kRouterTokens;
  const int nt = min(kRouterTokens, T - t0);
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int kb = w * (H / kRouterWaves), ke = kb + H / kRouterWaves;
  const size_t row = (size_t)H * ES;
  const char* wrow = wg + (size_t)e * row;
  const char* xrow = x + (size_t)t0 * row;
  float acc[kRouterTokens];
#pragma unroll
  for (int i = 0; i < kRouterTokens; i++) acc[i] = 0.f;
  for (int h0 = kb + lane * R::N; h0 < ke; h0 += kWave * R::N) {
    float w[R::N];
    R::load(wrow + (size_t)h0 * ES, w);
#pragma unroll
    for (int i = 0; i < kRouterTokens; i++) {
      if (i < nt) {
        float v[R::N];
        R::load(xrow + i * row + (size_t)h0 * ES, v);
#pragma unroll
        for (int q = 0; q < R::N; q++) acc[i] = fmaf(v[q], w[q], acc[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kRouterTokens; i++) {
    if (i < nt) {
      const float s = wave_sum(acc[i]);
      if (lane == 0) part[w][i] = s;
    }
  }
  __syncthreads();
  if (threadIdx.x < nt) {
    float s = part[0][threadIdx.x];
#pragma unroll
    for (int q = 1; q < kRouterWaves; q++) s += part[q][threadIdx.x];
    logits[(size_t)(t0 + threadIdx.x) * E + e] = s;
  }
}

// The token tiles of the tiled path: tile i covers tokens [64 i, 64 i + 64)
// of the single "expert" 0.
__global__ __launch_bounds__(256) void router_tiles_kernel(int T, Tile* __restrict__ tiles,
                                                           int32_t* num_tiles) {
  const int n = (T + kRouterBM - 1) / kRouterBM;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    Tile tl;
    tl.e = 0;
    tl.p0 = i * kRouterBM;
    tl.mt = min(kRouterBM, T - tl.p0);
    tl.pad = 0;
    tiles[i] = tl;
  }
  if (threadIdx.x == 0) *num_tiles = n;
}

bool router_uses_tiles(int mode, int T, int E) {
  return mode != MOE_F32 && E % 128 == 0 && T >= 4 * kRouterBM;
}

hipError_t launch_router_logits(int mode, const void* x, const void* wg, int T, int H, int E,
                                float* logits, Tile* tiles, int32_t* num_tiles, int max_tiles,
                                hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const char* xb = reinterpret_cast<const char*>(x);
  const char* wb = reinterpret_cast<const char*>(wg);
  if (router_uses_tiles(mode, T, E)) {
    router_tiles_kernel<<<1, 256, 0, st>>>(T, tiles, num_tiles);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // wg takes the weight side of the down-projection kernel: E output
    // features (its "H"), reduction length H (its "I"); bf16, no scales
    return launch_w2_tiles(MOE_BF16, kRouterBM, xb, wb, nullptr, tiles, num_tiles, max_tiles, E,
                           H, nullptr, logits, false, nullptr, nullptr, st);
  }
  const dim3 grid(E, (T + kRouterTokens - 1) / kRouterTokens);
  if (mode == MOE_F32)
    router_small_kernel<MOE_F32><<<grid, kRouterWaves * 64, 0, st>>>(xb, wb, T, H, E, logits);
  else
    router_small_kernel<MOE_BF16><<<grid, kRouterWaves * 64, 0, st>>>(xb, wb, T, H, E, logits);
  return hipGetLastError();
}

}  // namespace moe
