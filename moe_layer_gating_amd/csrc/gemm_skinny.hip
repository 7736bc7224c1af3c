// gemm_skinny.hip -- grouped expert GEMMs for few tokens per expert, with the
// expert weight rows on the MFMA row side ("swap-AB").
//
// With few tokens per expert the GEMM is a stream of expert weights.  On
// Hopper the token dimension would leave WGMMA's fixed 64-row side idle, so
// the operands are swapped and the large expert dimension takes that side
// (codebridge-ai.com, "aws-moe-kernel-wgmma-triton-ttft", section "1. Matrix
// swap"; readmex.ai, "Swap-AB for WGMMA utilization"; modelsatwork.news,
// "The three changes").  CDNA4 has no fixed 64-row side, but the same
// orientation is what makes gfx950 MFMA fit this shape: a 16x16 MFMA takes
// 16 weight rows on its row side and up to 16 tokens on its column side, so
// every weight byte is loaded once, by one lane, as part of a coalesced
// 16-byte load, and the token operand is the small one.
//
// Work decomposition: a block (4 waves) owns 16 weight rows of one expert
// for one tile of <= 16 sorted positions (one token-tile of the tile list)
// and the whole reduction dimension K; the 4 waves split K, reduce their
// 16x16 partial products through LDS in a fixed order, and the block
// applies the epilogue:
//   w13: rows 0-7 are gate rows n0..n0+7, rows 8-15 the matching up rows, so
//        the SwiGLU h = silu(c*g) * (c*u) is formed inside the block;
//   w2 : 16 output features of y, scaled by the FP8 dequantisation factor.
// Scales are applied to the fp32 accumulators in the epilogue (agentic-
// affairs.com, "Triton improves the FP8 execution path": scaling and the
// matrix multiplication in one pass).
//
// Operand layouts inside one MFMA (lane l, r = l % 16, g = l / 16):
//   A (weights): lane holds row r, a run of K values picked by g;
//   B (tokens) : lane holds token column r, the same run of K values;
//   C          : lane holds column r, rows 4g .. 4g+3.
// Because A and B use the same K assignment, the K order inside a step is a
// free choice; each lane loads a contiguous 16- or 32-byte run so that the
// 4 lanes of a row cover 64 (bf16/fp32) or 128 (FP8) contiguous bytes.
#include "moe_common.h"

namespace moe {

template <int MODE>
struct Step;

// bf16: one v_mfma_f32_16x16x32_bf16 per step; 8 bf16 (16 B) per lane.
template <>
struct Step<MOE_BF16> {
  static constexpr int KS = 32;     // K elements per step
  static constexpr int LANE_K = 8;  // K elements per lane per step
  static constexpr int ES = 2;      // bytes per element
  typedef i32x4 Frag;
  static __device__ __forceinline__ Frag load(const char* p) {
    return *reinterpret_cast<const i32x4*>(p);
  }
  static __device__ __forceinline__ Frag zero() { return i32x4{0, 0, 0, 0}; }
  static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// FP8 e4m3: one v_mfma_scale_f32_16x16x128_f8f6f4 (format e4m3 on both
// sides, unit block scales) per step; 32 codes (32 B) per lane.
template <>
struct Step<MOE_FP8_E4M3> {
  static constexpr int KS = 128;
  static constexpr int LANE_K = 32;
  static constexpr int ES = 1;
  typedef i32x8 Frag;
  static __device__ __forceinline__ Frag load(const char* p) {
    i32x4 lo = *reinterpret_cast<const i32x4*>(p);
    i32x4 hi = *reinterpret_cast<const i32x4*>(p + 16);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  static __device__ __forceinline__ Frag zero() { return i32x8{0, 0, 0, 0, 0, 0, 0, 0}; }
  static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    // scale operands: E8M0 exponent 127 = 2^0 for both A and B
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// fp32: four v_mfma_f32_16x16x4_f32 per step; 4 floats (16 B) per lane,
// the i-th MFMA of the step uses the lane's i-th float.
template <>
struct Step<MOE_F32> {
  static constexpr int KS = 16;
  static constexpr int LANE_K = 4;
  static constexpr int ES = 4;
  typedef i32x4 Frag;
  static __device__ __forceinline__ Frag load(const char* p) {
    return *reinterpret_cast<const i32x4*>(p);
  }
  static __device__ __forceinline__ Frag zero() { return i32x4{0, 0, 0, 0}; }
  static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
#pragma unroll
    for (int i = 0; i < 4; i++)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a[i]), __int_as_float(b[i]), c, 0, 0,
                                               0);
    return c;
  }
};

template <int MODE>
constexpr int unroll_for() {
  return MODE == MOE_FP8_E4M3 ? 4 : 8;
}

// Partial product of one wave: A rows `arow` (this lane's weight row), B row
// `brow` (this lane's token row, or nullptr for an empty column), over the
// wave's steps [s0, s1).
template <int MODE>
__device__ __forceinline__ f32x4 wave_dot(const char* __restrict__ arow, const char* __restrict__ brow,
                                          int s0, int s1, int g) {
  typedef Step<MODE> S;
  constexpr int U = unroll_for<MODE>();
  constexpr int STEP_BYTES = S::KS * S::ES;
  const int lane_off = g * S::LANE_K * S::ES;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int s = s0;
  for (; s + U <= s1; s += U) {
    typename S::Frag a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; u++) a[u] = S::load(arow + (size_t)(s + u) * STEP_BYTES + lane_off);
#pragma unroll
    for (int u = 0; u < U; u++)
      b[u] = brow ? S::load(brow + (size_t)(s + u) * STEP_BYTES + lane_off) : S::zero();
#pragma unroll
    for (int u = 0; u < U; u++) acc = S::mma(a[u], b[u], acc);
  }
  for (; s < s1; s++) {
    typename S::Frag a = S::load(arow + (size_t)s * STEP_BYTES + lane_off);
    typename S::Frag b = brow ? S::load(brow + (size_t)s * STEP_BYTES + lane_off) : S::zero();
    acc = S::mma(a, b, acc);
  }
  return acc;
}

__device__ __forceinline__ float act_scale_from_bits(const uint32_t* bits) {
  float a = __uint_as_float(*bits);
  return a > 0.f ? a / 448.0f : 1.0f;
}

// Reduce the 4 waves' 16x16 partials; result in fin[row][col].
__device__ __forceinline__ void block_reduce_16x16(f32x4 acc, float (*red)[16][16],
                                                   float (*fin)[16]) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int col = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; i++) red[w][4 * g + i][col] = acc[i];
  __syncthreads();
  const int row = threadIdx.x >> 4, c = threadIdx.x & 15;
  fin[row][c] = ((red[0][row][c] + red[1][row][c]) + red[2][row][c]) + red[3][row][c];
  __syncthreads();
}

// ------------------------------------------------------------------- w13
template <int MODE>
__global__ __launch_bounds__(256) void w13_swiglu_skinny(
    const char* __restrict__ b, const char* __restrict__ w13, const float* __restrict__ w13_scale,
    const int32_t* __restrict__ sorted_ids, const Tile* __restrict__ tiles,
    const Ctrl* __restrict__ ctrl, int H, int I, int k, const uint32_t* act_amax_bits,
    void* __restrict__ h, uint32_t* amax_h_bits) {
  typedef Step<MODE> S;
  __shared__ float red[4][16][16];
  __shared__ float fin[16][16];
  __shared__ float bmax[4];
  const int n_rt = I / 8;
  const int tile_idx = blockIdx.x / n_rt;
  const int rt = blockIdx.x - tile_idx * n_rt;
  if (tile_idx >= ctrl->num_tiles) return;
  const Tile tl = tiles[tile_idx];
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = rt * 8;
  // this lane's weight row: gate rows n0..n0+7, then up rows I+n0..I+n0+7
  const int wrow = (r < 8) ? (n0 + r) : (I + n0 + r - 8);
  const char* arow = w13 + ((size_t)tl.e * 2 * I + wrow) * (size_t)H * S::ES;
  const char* brow = nullptr;
  if (r < tl.mt) {
    int tok = sorted_ids[tl.p0 + r] / k;
    brow = b + (size_t)tok * H * S::ES;
  }
  const int n_steps = H / S::KS;
  const int s0 = (w * n_steps) / 4, s1 = ((w + 1) * n_steps) / 4;
  f32x4 acc = wave_dot<MODE>(arow, brow, s0, s1, g);
  block_reduce_16x16(acc, red, fin);

  float c = 1.0f;
  if (MODE == MOE_FP8_E4M3) c = act_scale_from_bits(act_amax_bits) * w13_scale[tl.e];
  float hmax = 0.f;
  if (threadIdx.x < 128) {
    const int j = threadIdx.x >> 3, rr = threadIdx.x & 7;
    if (j < tl.mt) {
      float gv = fin[rr][j], uv = fin[rr + 8][j];
      if (MODE == MOE_FP8_E4M3) {
        gv *= c;
        uv *= c;
      }
      float hv = gv / (1.0f + expf(-gv)) * uv;
      size_t o = (size_t)(tl.p0 + j) * I + n0 + rr;
      if (MODE == MOE_F32) {
        reinterpret_cast<float*>(h)[o] = hv;
      } else {
        uint16_t hb = f32_to_bf16(hv);
        reinterpret_cast<uint16_t*>(h)[o] = hb;
        hmax = fabsf(bf16_to_f32(hb));
      }
    }
  }
  if (MODE == MOE_FP8_E4M3) {
    hmax = wave_max(hmax);
    if (lane == 0) bmax[w] = hmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      float m = fmaxf(fmaxf(bmax[0], bmax[1]), fmaxf(bmax[2], bmax[3]));
      atomicMax(amax_h_bits, __float_as_uint(m));
    }
  }
}

// -------------------------------------------------------------------- w2
template <int MODE>
__global__ __launch_bounds__(256) void w2_skinny(const char* __restrict__ b,
                                                 const char* __restrict__ w2,
                                                 const float* __restrict__ w2_scale,
                                                 const Tile* __restrict__ tiles,
                                                 const Ctrl* __restrict__ ctrl, int H, int I,
                                                 const uint32_t* act_amax_bits,
                                                 float* __restrict__ y) {
  typedef Step<MODE> S;
  __shared__ float red[4][16][16];
  __shared__ float fin[16][16];
  const int n_rt = H / 16;
  const int tile_idx = blockIdx.x / n_rt;
  const int rt = blockIdx.x - tile_idx * n_rt;
  if (tile_idx >= ctrl->num_tiles) return;
  const Tile tl = tiles[tile_idx];
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int m0 = rt * 16;
  const char* arow = w2 + ((size_t)tl.e * H + m0 + r) * (size_t)I * S::ES;
  const char* brow = (r < tl.mt) ? b + (size_t)(tl.p0 + r) * I * S::ES : nullptr;
  const int n_steps = I / S::KS;
  const int s0 = (w * n_steps) / 4, s1 = ((w + 1) * n_steps) / 4;
  f32x4 acc = wave_dot<MODE>(arow, brow, s0, s1, g);
  block_reduce_16x16(acc, red, fin);
  float c = 1.0f;
  if (MODE == MOE_FP8_E4M3) c = act_scale_from_bits(act_amax_bits) * w2_scale[tl.e];
  const int j = threadIdx.x >> 4, mm = threadIdx.x & 15;
  if (j < tl.mt) {
    float v = fin[mm][j];
    if (MODE == MOE_FP8_E4M3) v *= c;
    y[(size_t)(tl.p0 + j) * H + m0 + mm] = v;
  }
}

hipError_t launch_w13_swiglu(int mode, const void* b, const void* w13, const float* w13_scale,
                             const int32_t* sorted_ids, const Tile* tiles, const Ctrl* ctrl,
                             int max_tiles, int H, int I, int k, const uint32_t* act_amax_bits,
                             void* h, uint32_t* amax_h_bits, hipStream_t st) {
  long blocks = (long)max_tiles * (I / 8);
  if (blocks <= 0) return hipSuccess;
  const char* bb = reinterpret_cast<const char*>(b);
  const char* ww = reinterpret_cast<const char*>(w13);
  switch (mode) {
    case MOE_F32:
      w13_swiglu_skinny<MOE_F32><<<blocks, 256, 0, st>>>(bb, ww, w13_scale, sorted_ids, tiles, ctrl,
                                                         H, I, k, act_amax_bits, h, amax_h_bits);
      break;
    case MOE_BF16:
      w13_swiglu_skinny<MOE_BF16><<<blocks, 256, 0, st>>>(bb, ww, w13_scale, sorted_ids, tiles,
                                                          ctrl, H, I, k, act_amax_bits, h,
                                                          amax_h_bits);
      break;
    default:
      w13_swiglu_skinny<MOE_FP8_E4M3><<<blocks, 256, 0, st>>>(bb, ww, w13_scale, sorted_ids, tiles,
                                                              ctrl, H, I, k, act_amax_bits, h,
                                                              amax_h_bits);
  }
  return hipGetLastError();
}

hipError_t launch_w2(int mode, const void* b, const void* w2, const float* w2_scale,
                     const Tile* tiles, const Ctrl* ctrl, int max_tiles, int H, int I,
                     const uint32_t* act_amax_bits, float* y, hipStream_t st) {
  long blocks = (long)max_tiles * (H / 16);
  if (blocks <= 0) return hipSuccess;
  const char* bb = reinterpret_cast<const char*>(b);
  const char* ww = reinterpret_cast<const char*>(w2);
  switch (mode) {
    case MOE_F32:
      w2_skinny<MOE_F32><<<blocks, 256, 0, st>>>(bb, ww, w2_scale, tiles, ctrl, H, I,
                                                 act_amax_bits, y);
      break;
    case MOE_BF16:
      w2_skinny<MOE_BF16><<<blocks, 256, 0, st>>>(bb, ww, w2_scale, tiles, ctrl, H, I,
                                                  act_amax_bits, y);
      break;
    default:
      w2_skinny<MOE_FP8_E4M3><<<blocks, 256, 0, st>>>(bb, ww, w2_scale, tiles, ctrl, H, I,
                                                      act_amax_bits, y);
  }
  return hipGetLastError();
}

}  // namespace moe
