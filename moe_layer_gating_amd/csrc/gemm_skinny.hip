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
// Work decomposition: a row group is 16 weight rows of one expert for one
// tile of <= 16 sorted positions (one entry of the tile list), over the whole
// reduction dimension K.  A block's NW waves all take the same row group and
// split K; their 16x16 partial products are added through LDS in a fixed
// order.  The epilogue then forms
//   w13: the SwiGLU h = silu(c*g) * (c*u) (gate and up rows interleaved);
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

// FP8 codes on the bf16 MFMA (kFp8ViaBf16): the same 32 codes per lane as
// Step<MOE_FP8_E4M3>, widened to bf16; the u-th of four
// v_mfma_f32_16x16x32_bf16 takes the lane's codes 8u .. 8u+7 of A and of B,
// so a step sums the same 128 products.
template <>
struct Step<kFp8ViaBf16> {
  static constexpr int KS = 128;
  static constexpr int LANE_K = 32;
  static constexpr int ES = 1;
  typedef i32x8 Frag;
  static __device__ __forceinline__ Frag load(const char* p) {
    return Step<MOE_FP8_E4M3>::load(p);
  }
  static __device__ __forceinline__ Frag zero() { return Step<MOE_FP8_E4M3>::zero(); }
  static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
#pragma unroll
    for (int u = 0; u < 4; u++)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, e4m3x8_to_bf16x8(a[2 * u], a[2 * u + 1])),
          __builtin_bit_cast(bf16x8, e4m3x8_to_bf16x8(b[2 * u], b[2 * u + 1])), c, 0, 0, 0);
    return c;
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

// Steps of loads issued ahead of their MFMAs: 128 bytes per lane in every mode
// (deeper unrolls and non-temporal weight loads both measured slower on the
// decode shapes).
template <int MODE>
constexpr int unroll_for() {
  return is_fp8(MODE) ? 4 : 8;
}

// Partial product of one wave: A row `arow` (this lane's weight row), B row
// `brow` (this lane's token row, or nullptr for an empty column), over the
// wave's steps [s0, s1).  U steps of loads are issued before their MFMAs.
template <int MODE, int U>
__device__ __forceinline__ f32x4 wave_dot(const char* __restrict__ arow,
                                          const char* __restrict__ brow,
                                          int s0, int s1, int g) {
  typedef Step<MODE> S;
  constexpr int STEP_BYTES = S::KS * S::ES;
  const int lane_off = g * S::LANE_K * S::ES;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int s = s0;
  for (; s + U <= s1; s += U) {
    typename S::Frag a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      a[u] = S::load(arow + (size_t)(s + u) * STEP_BYTES + lane_off);
    }
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

// Sum the NW partial 16x16 products of the block's waves in a fixed order
// ((w0 + w1) + w2) + ...; the result is valid in wave 0 only.
template <int NW>
__device__ __forceinline__ f32x4 block_reduce(f32x4 acc, float (*red)[64][4]) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
  if (w > 0) {
#pragma unroll
    for (int i = 0; i < 4; i++) red[w - 1][lane][i] = acc[i];
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int q = 1; q < NW; q++)
#pragma unroll
      for (int i = 0; i < 4; i++) acc[i] += red[q - 1][lane][i];
  }
  return acc;
}

// Raise *amax_bits to v (a non-negative float) unless it is already at least
// v: reading first keeps most waves off the single contended address; a stale
// read only costs an atomic that changes nothing.
__device__ __forceinline__ void amax_update(uint32_t* amax_bits, float v) {
  const uint32_t bits = __float_as_uint(v);
  if (bits > __atomic_load_n(amax_bits, __ATOMIC_RELAXED)) atomicMax(amax_bits, bits);
}

// ------------------------------------------------------------------- w13
// Block = NW waves on one row group of 8 gate rows n0..n0+7 and the 8
// matching up rows, interleaved on the MFMA row side: MFMA row 2i is gate row
// n0+i, row 2i+1 up row I+n0+i.  The accumulator rows a lane holds
// (4g..4g+3) are then gate/up/gate/up of features n0+2g and n0+2g+1, so the
// SwiGLU is formed inside the lane.  The NW waves split K.
template <int MODE, int NW, int U = unroll_for<MODE>()>
__global__ __launch_bounds__(NW * 64) void w13_swiglu_skinny(
    const char* __restrict__ b, const char* __restrict__ w13, const float* __restrict__ w13_scale,
    const int32_t* __restrict__ sorted_ids, const Tile* __restrict__ tiles,
    const Ctrl* __restrict__ ctrl, int H, int I, int k, const uint32_t* act_amax_bits,
    void* __restrict__ h, uint32_t* amax_h_bits) {
  typedef Step<MODE> S;
  __shared__ float red[NW - 1][64][4];
  const int blocks_per_tile = I / 8;
  const int tile_idx = blockIdx.x / blocks_per_tile;
  const int rb = blockIdx.x - tile_idx * blocks_per_tile;
  if (tile_idx >= ctrl->num_tiles) return;
  const Tile tl = tiles[tile_idx];
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = rb * 8;
  const int wrow = (r & 1) ? (I + n0 + (r >> 1)) : (n0 + (r >> 1));
  const char* arow = w13 + ((size_t)tl.e * 2 * I + wrow) * (size_t)H * S::ES;
  const char* brow = nullptr;
  if (r < tl.mt) {
    int tok = sorted_ids[tl.p0 + r] / k;
    brow = b + (size_t)tok * H * S::ES;
  }
  const int n_steps = H / S::KS;
  const int s0 = (w * n_steps) / NW, s1 = ((w + 1) * n_steps) / NW;
  f32x4 acc = wave_dot<MODE, U>(arow, brow, s0, s1, g);
  acc = block_reduce<NW>(acc, red);
  if (w != 0) return;

  float c = 1.0f;
  if (is_fp8(MODE)) c = act_scale_from_bits(act_amax_bits) * w13_scale[tl.e];
  float hmax = 0.f;
  if (r < tl.mt) {
    float hv[2];
#pragma unroll
    for (int q = 0; q < 2; q++) {
      float gv = acc[2 * q], uv = acc[2 * q + 1];
      if (is_fp8(MODE)) {
        gv *= c;
        uv *= c;
      }
      hv[q] = gv / (1.0f + expf(-gv)) * uv;
    }
    size_t o = (size_t)(tl.p0 + r) * I + n0 + 2 * g;
    if (MODE == MOE_F32) {
      *reinterpret_cast<float2*>(reinterpret_cast<float*>(h) + o) = make_float2(hv[0], hv[1]);
    } else {
      uint16_t h0 = f32_to_bf16(hv[0]), h1 = f32_to_bf16(hv[1]);
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(h) + o) =
          (uint32_t)h0 | ((uint32_t)h1 << 16);
      hmax = fmaxf(fabsf(bf16_to_f32(h0)), fabsf(bf16_to_f32(h1)));
    }
  }
  if (is_fp8(MODE)) {
    hmax = wave_max(hmax);
    if (lane == 0) amax_update(amax_h_bits, hmax);
  }
}

// -------------------------------------------------------------------- w2
// Block = NW waves on one row group of 16 output features m0..m0+15, splitting
// K.  A lane's accumulator rows 4g..4g+3 are 4 consecutive features of its
// token column: one 16-byte store of y.
template <int MODE, int NW, int U = unroll_for<MODE>()>
__global__ __launch_bounds__(NW * 64) void w2_skinny(const char* __restrict__ b,
                                                     const char* __restrict__ w2,
                                                     const float* __restrict__ w2_scale,
                                                     const Tile* __restrict__ tiles,
                                                     const Ctrl* __restrict__ ctrl, int H, int I,
                                                     const uint32_t* act_amax_bits,
                                                     float* __restrict__ y) {
  typedef Step<MODE> S;
  __shared__ float red[NW - 1][64][4];
  const int blocks_per_tile = H / 16;
  const int tile_idx = blockIdx.x / blocks_per_tile;
  const int rb = blockIdx.x - tile_idx * blocks_per_tile;
  if (tile_idx >= ctrl->num_tiles) return;
  const Tile tl = tiles[tile_idx];
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int m0 = rb * 16;
  const char* arow = w2 + ((size_t)tl.e * H + m0 + r) * (size_t)I * S::ES;
  const char* brow = (r < tl.mt) ? b + (size_t)(tl.p0 + r) * I * S::ES : nullptr;
  const int n_steps = I / S::KS;
  const int s0 = (w * n_steps) / NW, s1 = ((w + 1) * n_steps) / NW;
  f32x4 acc = wave_dot<MODE, U>(arow, brow, s0, s1, g);
  acc = block_reduce<NW>(acc, red);
  if (w != 0 || r >= tl.mt) return;
  if (MODE == MOE_FP8_E4M3) acc *= act_scale_from_bits(act_amax_bits) * w2_scale[tl.e];
  *reinterpret_cast<f32x4*>(y + (size_t)(tl.p0 + r) * H + m0 + 4 * g) = acc;
}

// Waves per block (all splitting K over one row group).  A block's waves
// stream the same 16 rows at different K offsets, so the block's concurrent
// loads fall in the same few DRAM pages.
template <int MODE>
constexpr int waves_w13() {
  return 4;
}
// The bf16 down projection (K = I, the longest rows) measured fastest with 16
// waves over 4 steps of loads each.
template <int MODE>
constexpr int waves_w2() {
  return MODE == MOE_BF16 ? 16 : 4;
}
template <int MODE>
constexpr int unroll_w2() {
  return MODE == MOE_BF16 ? 4 : unroll_for<MODE>();
}

template <int MODE>
static void launch_w13_mode(long max_tiles, const char* b, const char* w13, const float* w13_scale,
                            const int32_t* sorted_ids, const Tile* tiles, const Ctrl* ctrl, int H,
                            int I, int k, const uint32_t* act_amax_bits, void* h,
                            uint32_t* amax_h_bits, hipEvent_t e0, hipEvent_t e1, hipStream_t st) {
  constexpr int NW = waves_w13<MODE>();
  const long blocks = max_tiles * (I / 8);
  launch_on(w13_swiglu_skinny<MODE, NW>, dim3(blocks), dim3(NW * 64), st, e0, e1, b, w13,
            w13_scale, sorted_ids, tiles, ctrl, H, I, k, act_amax_bits, h, amax_h_bits);
}

template <int MODE>
static void launch_w2_mode(long max_tiles, const char* b, const char* w2, const float* w2_scale,
                           const Tile* tiles, const Ctrl* ctrl, int H, int I,
                           const uint32_t* act_amax_bits, float* y, hipEvent_t e0, hipEvent_t e1,
                           hipStream_t st) {
  constexpr int NW = waves_w2<MODE>();
  const long blocks = max_tiles * (H / 16);
  launch_on(w2_skinny<MODE, NW, unroll_w2<MODE>()>, dim3(blocks), dim3(NW * 64), st, e0, e1, b,
            w2, w2_scale, tiles,
            ctrl, H, I, act_amax_bits, y);
}

hipError_t launch_w13_swiglu(int mode, const void* b, const void* w13, const float* w13_scale,
                             const int32_t* sorted_ids, const Tile* tiles, const Ctrl* ctrl,
                             int max_tiles, int H, int I, int k, const uint32_t* act_amax_bits,
                             void* h, uint32_t* amax_h_bits, hipEvent_t e0, hipEvent_t e1,
                             hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  const char* bb = reinterpret_cast<const char*>(b);
  const char* ww = reinterpret_cast<const char*>(w13);
  if (mode == MOE_F32)
    launch_w13_mode<MOE_F32>(max_tiles, bb, ww, w13_scale, sorted_ids, tiles, ctrl, H, I, k,
                             act_amax_bits, h, amax_h_bits, e0, e1, st);
  else if (mode == MOE_BF16)
    launch_w13_mode<MOE_BF16>(max_tiles, bb, ww, w13_scale, sorted_ids, tiles, ctrl, H, I, k,
                              act_amax_bits, h, amax_h_bits, e0, e1, st);
  else
    launch_w13_mode<kFp8ViaBf16>(max_tiles, bb, ww, w13_scale, sorted_ids, tiles, ctrl, H, I, k,
                                 act_amax_bits, h, amax_h_bits, e0, e1, st);
  return hipGetLastError();
}

hipError_t launch_w2(int mode, const void* b, const void* w2, const float* w2_scale,
                     const Tile* tiles, const Ctrl* ctrl, int max_tiles, int H, int I,
                     const uint32_t* act_amax_bits, float* y, hipEvent_t e0, hipEvent_t e1,
                     hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  const char* bb = reinterpret_cast<const char*>(b);
  const char* ww = reinterpret_cast<const char*>(w2);
  if (mode == MOE_F32)
    launch_w2_mode<MOE_F32>(max_tiles, bb, ww, w2_scale, tiles, ctrl, H, I, act_amax_bits, y, e0,
                            e1, st);
  else if (mode == MOE_BF16)
    launch_w2_mode<MOE_BF16>(max_tiles, bb, ww, w2_scale, tiles, ctrl, H, I, act_amax_bits, y, e0,
                             e1, st);
  else
    launch_w2_mode<MOE_FP8_E4M3>(max_tiles, bb, ww, w2_scale, tiles, ctrl, H, I, act_amax_bits, y,
                                 e0, e1, st);
  return hipGetLastError();
}

}  // namespace moe
