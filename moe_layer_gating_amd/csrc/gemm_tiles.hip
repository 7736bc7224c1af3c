// gemm_tiles.hip -- grouped expert GEMMs for many tokens per expert (prefill
// and mixed batches), FP8 e4m3 or bf16, with LDS-staged operand tiles.
//
// When an expert receives tens to thousands of tokens, its weights can be
// reused from on-chip memory across many tokens and the GEMM becomes a real
// 2-D tiled contraction.  A block owns a 128 (weight rows) x BM (sorted
// positions of one expert) output tile and walks the reduction dimension K in
// 128-byte stages (128 FP8 codes or 64 bf16 values per row), double-buffered
// in LDS.  Four waves split the tile 2 x 2; each wave holds a 64 x BM/2
// accumulator of 16x16 MFMA tiles.  Both operands keep K contiguous in HBM,
// so every stage loads whole 128-byte lines: 8 lanes per row.
//
// LDS layout: row r of a 128-byte-wide stage keeps its 16-byte chunk c at
// slot c ^ swz(r), swz(r) = (r ^ (r >> 3)) & 7.  Eight consecutive rows read
// at one chunk index then hit eight different slots, as do sixteen
// consecutive rows counted over two 128-byte bank rows, so neither the
// stores nor the MFMA fragment reads conflict in the LDS banks.
//
// The expert rows sit on the MFMA row side and the tokens on the column side,
// as in the decode kernels (codebridge-ai.com, "aws-moe-kernel-wgmma-triton-
// ttft", section "1. Matrix swap"), and the dequantisation scales are applied
// to the fp32 accumulators in the epilogue (agentic-affairs.com, "Triton
// improves the FP8 execution path").
//
// Launch order: block b takes tile b / NB and weight-row block b % NB, with
// NB = (rows of the weight matrix) / 128.  Blocks are dealt to the 8 XCDs
// round-robin, so when NB is a multiple of 8 a given weight-row block of an
// expert always runs on the same XCD and its reuse across the expert's
// token tiles is served by that XCD's L2.
#include "moe_common.h"

namespace moe {

constexpr int kTileN = 128;  // weight rows per block tile
constexpr int kStageB = 128;  // bytes of K per row per stage

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// MFMA work of one 128-byte K stage for one 16x16 output tile.
template <int MODE>
struct TileMma;

// FP8: one v_mfma_scale_f32_16x16x128_f8f6f4; the lane's 32 bytes are
// chunks 2g and 2g+1 of its row.
template <>
struct TileMma<MOE_FP8_E4M3> {
  typedef i32x8 Frag;
  static constexpr int NFRAG = 1;  // fragments per stage
  static __device__ __forceinline__ Frag read(const char* row, int sw, int g, int f) {
    (void)f;
    i32x4 lo = *reinterpret_cast<const i32x4*>(row + (((2 * g) ^ sw) << 4));
    i32x4 hi = *reinterpret_cast<const i32x4*>(row + (((2 * g + 1) ^ sw) << 4));
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// bf16: two v_mfma_f32_16x16x32_bf16 per stage; step f uses chunk 4f+g.
template <>
struct TileMma<MOE_BF16> {
  typedef i32x4 Frag;
  static constexpr int NFRAG = 2;
  static __device__ __forceinline__ Frag read(const char* row, int sw, int g, int f) {
    return *reinterpret_cast<const i32x4*>(row + (((4 * f + g) ^ sw) << 4));
  }
  static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// Main loop shared by both projections.  a_rows / b_rows: this thread's rows
// to stage (4 weight rows, BM/32 token rows), each pointing at K offset 0 of
// the row plus the thread's chunk (t & 7) * 16.  Accumulates into acc.
template <int MODE, int BM>
__device__ __forceinline__ void tile_mainloop(const char* const* a_rows, const char* const* b_rows,
                                              int n_stages, char* lds, f32x4 (*acc)[BM / 32]) {
  typedef TileMma<MODE> M;
  constexpr int A_BYTES = kTileN * kStageB;
  constexpr int B_BYTES = BM * kStageB;
  constexpr int BUF = A_BYTES + B_BYTES;
  constexpr int NA = kTileN / 32, NB = BM / 32;  // rows staged per thread
  constexpr int MT = BM / 32;                    // 16-column tiles per wave
  const int t = threadIdx.x;
  const int lane = lane_id(), w = t / kWave;
  const int r16 = lane & 15, g = lane >> 4;
  const int wn = w >> 1, wm = w & 1;
  const int c = t & 7, r0 = t >> 3;

  // store slots of this thread's staged rows
  int a_slot[NA], b_slot[NB];
#pragma unroll
  for (int i = 0; i < NA; i++) {
    int r = r0 + 32 * i;
    a_slot[i] = r * kStageB + ((c ^ swz(r)) << 4);
  }
#pragma unroll
  for (int i = 0; i < NB; i++) {
    int r = r0 + 32 * i;
    b_slot[i] = A_BYTES + r * kStageB + ((c ^ swz(r)) << 4);
  }
  // read rows of this lane's fragments
  int a_off[4], a_sw[4], b_off[MT], b_sw[MT];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    int r = wn * 64 + i * 16 + r16;
    a_off[i] = r * kStageB;
    a_sw[i] = swz(r);
  }
#pragma unroll
  for (int j = 0; j < MT; j++) {
    int r = wm * (BM / 2) + j * 16 + r16;
    b_off[j] = A_BYTES + r * kStageB;
    b_sw[j] = swz(r);
  }

  i32x4 ra[NA], rb[NB];
#pragma unroll
  for (int i = 0; i < NA; i++) ra[i] = *reinterpret_cast<const i32x4*>(a_rows[i]);
#pragma unroll
  for (int i = 0; i < NB; i++) rb[i] = *reinterpret_cast<const i32x4*>(b_rows[i]);
#pragma unroll
  for (int i = 0; i < NA; i++) *reinterpret_cast<i32x4*>(lds + a_slot[i]) = ra[i];
#pragma unroll
  for (int i = 0; i < NB; i++) *reinterpret_cast<i32x4*>(lds + b_slot[i]) = rb[i];
  __syncthreads();

  for (int kt = 0; kt < n_stages; kt++) {
    const char* cur = lds + (kt & 1) * BUF;
    char* nxt = lds + ((kt + 1) & 1) * BUF;
    const bool more = kt + 1 < n_stages;
    if (more) {
      const size_t off = (size_t)(kt + 1) * kStageB;
#pragma unroll
      for (int i = 0; i < NA; i++) ra[i] = *reinterpret_cast<const i32x4*>(a_rows[i] + off);
#pragma unroll
      for (int i = 0; i < NB; i++) rb[i] = *reinterpret_cast<const i32x4*>(b_rows[i] + off);
    }
#pragma unroll
    for (int f = 0; f < M::NFRAG; f++) {
      typename M::Frag fa[4], fb[MT];
#pragma unroll
      for (int i = 0; i < 4; i++) fa[i] = M::read(cur + a_off[i], a_sw[i], g, f);
#pragma unroll
      for (int j = 0; j < MT; j++) fb[j] = M::read(cur + b_off[j], b_sw[j], g, f);
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < MT; j++) acc[i][j] = M::mma(fa[i], fb[j], acc[i][j]);
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < NA; i++) *reinterpret_cast<i32x4*>(nxt + a_slot[i]) = ra[i];
#pragma unroll
      for (int i = 0; i < NB; i++) *reinterpret_cast<i32x4*>(nxt + b_slot[i]) = rb[i];
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------- w13
// Block rows: MFMA tile q (0..7) row 2i is gate feature nb*64 + 8q + i, row
// 2i+1 the matching up feature, so a lane's accumulator rows 4g..4g+3 hold
// gate/up/gate/up of features nb*64 + 8q + 2g and + 1.
template <int MODE, int BM>
__global__ __launch_bounds__(256) void w13_swiglu_tiles(
    const char* __restrict__ b, const char* __restrict__ w13, const float* __restrict__ w13_scale,
    const int32_t* __restrict__ sorted_ids, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, int H, int I, int k, const uint32_t* act_amax_bits,
    void* __restrict__ h, uint32_t* amax_h_bits) {
  constexpr int ES = MODE == MOE_FP8_E4M3 ? 1 : 2;
  constexpr int MT = BM / 32;
  __shared__ __attribute__((aligned(16))) char lds[2 * (kTileN + BM) * kStageB];
  const int NBLK = 2 * I / kTileN;
  const int tile_idx = blockIdx.x / NBLK;
  const int nb = blockIdx.x - tile_idx * NBLK;
  if (tile_idx >= *num_tiles) return;
  const Tile tl = tiles[tile_idx];
  const int t = threadIdx.x, c = t & 7, r0 = t >> 3;
  const size_t row_bytes = (size_t)H * ES;

  const char* a_rows[kTileN / 32];
#pragma unroll
  for (int i = 0; i < kTileN / 32; i++) {
    int R = r0 + 32 * i, q = R >> 4, rr = R & 15;
    int f = nb * 64 + q * 8 + (rr >> 1);
    int wrow = (rr & 1) ? I + f : f;
    a_rows[i] = w13 + ((size_t)tl.e * 2 * I + wrow) * row_bytes + c * 16;
  }
  const char* b_rows[BM / 32];
#pragma unroll
  for (int i = 0; i < BM / 32; i++) {
    int j = min(r0 + 32 * i, tl.mt - 1);
    int tok = sorted_ids[tl.p0 + j] / k;
    b_rows[i] = b + (size_t)tok * row_bytes + c * 16;
  }
  f32x4 acc[4][MT];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < MT; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  tile_mainloop<MODE, BM>(a_rows, b_rows, (int)(row_bytes / kStageB), lds, acc);

  const int lane = lane_id(), w = t / kWave;
  const int r16 = lane & 15, g = lane >> 4, wn = w >> 1, wm = w & 1;
  float cs = 1.0f;
  if (MODE == MOE_FP8_E4M3) {
    float a = __uint_as_float(*act_amax_bits);
    cs = (a > 0.f ? a / 448.0f : 1.0f) * w13_scale[tl.e];
  }
  float hmax = 0.f;
#pragma unroll
  for (int j = 0; j < MT; j++) {
    const int col = wm * (BM / 2) + j * 16 + r16;
    if (col < tl.mt) {
      uint16_t* hrow = reinterpret_cast<uint16_t*>(h) + (size_t)(tl.p0 + col) * I;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int f = nb * 64 + (wn * 4 + i) * 8 + 2 * g;
        float hv[2];
#pragma unroll
        for (int q = 0; q < 2; q++) {
          float gv = acc[i][j][2 * q], uv = acc[i][j][2 * q + 1];
          if (MODE == MOE_FP8_E4M3) {
            gv *= cs;
            uv *= cs;
          }
          hv[q] = gv / (1.0f + expf(-gv)) * uv;
        }
        uint16_t h0 = f32_to_bf16(hv[0]), h1 = f32_to_bf16(hv[1]);
        *reinterpret_cast<uint32_t*>(hrow + f) = (uint32_t)h0 | ((uint32_t)h1 << 16);
        hmax = fmaxf(hmax, fmaxf(fabsf(bf16_to_f32(h0)), fabsf(bf16_to_f32(h1))));
      }
    }
  }
  if (MODE == MOE_FP8_E4M3) {
    hmax = wave_max(hmax);
    if (lane == 0) {
      const uint32_t bits = __float_as_uint(hmax);
      if (bits > __atomic_load_n(amax_h_bits, __ATOMIC_RELAXED)) atomicMax(amax_h_bits, bits);
    }
  }
}

// -------------------------------------------------------------------- w2
template <int MODE, int BM>
__global__ __launch_bounds__(256) void w2_tiles(const char* __restrict__ b,
                                                const char* __restrict__ w2,
                                                const float* __restrict__ w2_scale,
                                                const Tile* __restrict__ tiles,
                                                const int32_t* __restrict__ num_tiles, int H, int I,
                                                const uint32_t* act_amax_bits,
                                                float* __restrict__ y) {
  constexpr int ES = MODE == MOE_FP8_E4M3 ? 1 : 2;
  constexpr int MT = BM / 32;
  __shared__ __attribute__((aligned(16))) char lds[2 * (kTileN + BM) * kStageB];
  const int NBLK = H / kTileN;
  const int tile_idx = blockIdx.x / NBLK;
  const int nb = blockIdx.x - tile_idx * NBLK;
  if (tile_idx >= *num_tiles) return;
  const Tile tl = tiles[tile_idx];
  const int t = threadIdx.x, c = t & 7, r0 = t >> 3;
  const size_t row_bytes = (size_t)I * ES;

  const char* a_rows[kTileN / 32];
#pragma unroll
  for (int i = 0; i < kTileN / 32; i++)
    a_rows[i] = w2 + ((size_t)tl.e * H + nb * kTileN + r0 + 32 * i) * row_bytes + c * 16;
  const char* b_rows[BM / 32];
#pragma unroll
  for (int i = 0; i < BM / 32; i++) {
    int j = min(r0 + 32 * i, tl.mt - 1);
    b_rows[i] = b + (size_t)(tl.p0 + j) * row_bytes + c * 16;
  }
  f32x4 acc[4][MT];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < MT; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  tile_mainloop<MODE, BM>(a_rows, b_rows, (int)(row_bytes / kStageB), lds, acc);

  const int lane = lane_id(), w = t / kWave;
  const int r16 = lane & 15, g = lane >> 4, wn = w >> 1, wm = w & 1;
  float cs = 1.0f;
  if (MODE == MOE_FP8_E4M3) {
    float a = __uint_as_float(*act_amax_bits);
    cs = (a > 0.f ? a / 448.0f : 1.0f) * w2_scale[tl.e];
  }
#pragma unroll
  for (int j = 0; j < MT; j++) {
    const int col = wm * (BM / 2) + j * 16 + r16;
    if (col < tl.mt) {
      float* yrow = y + (size_t)(tl.p0 + col) * H + nb * kTileN;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        f32x4 v = acc[i][j];
        if (MODE == MOE_FP8_E4M3) v *= cs;
        *reinterpret_cast<f32x4*>(yrow + (wn * 4 + i) * 16 + 4 * g) = v;
      }
    }
  }
}

template <int MODE>
static void launch_tiles_w13_mode(long max_tiles, const char* b, const char* w13,
                                  const float* w13_scale, const int32_t* sorted_ids,
                                  const Tile* tiles, const int32_t* num_tiles, int H, int I, int k,
                                  const uint32_t* act_amax_bits, void* h, uint32_t* amax_h_bits,
                                  hipStream_t st) {
  const long blocks = max_tiles * (2L * I / kTileN);
  w13_swiglu_tiles<MODE, kTilesBM><<<blocks, 256, 0, st>>>(
      b, w13, w13_scale, sorted_ids, tiles, num_tiles, H, I, k, act_amax_bits, h, amax_h_bits);
}

template <int MODE>
static void launch_tiles_w2_mode(long max_tiles, const char* b, const char* w2,
                                 const float* w2_scale, const Tile* tiles,
                                 const int32_t* num_tiles, int H, int I,
                                 const uint32_t* act_amax_bits, float* y, hipStream_t st) {
  const long blocks = max_tiles * (long)(H / kTileN);
  w2_tiles<MODE, kTilesBM><<<blocks, 256, 0, st>>>(b, w2, w2_scale, tiles, num_tiles, H, I,
                                                   act_amax_bits, y);
}

hipError_t launch_w13_tiles(int mode, const void* b, const void* w13, const float* w13_scale,
                            const int32_t* sorted_ids, const Tile* tiles,
                            const int32_t* num_tiles, int max_tiles, int H, int I, int k,
                            const uint32_t* act_amax_bits, void* h, uint32_t* amax_h_bits,
                            hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  const char* bb = reinterpret_cast<const char*>(b);
  const char* ww = reinterpret_cast<const char*>(w13);
  if (mode == MOE_BF16)
    launch_tiles_w13_mode<MOE_BF16>(max_tiles, bb, ww, w13_scale, sorted_ids, tiles, num_tiles, H,
                                    I, k, act_amax_bits, h, amax_h_bits, st);
  else if (mode == MOE_FP8_E4M3)
    launch_tiles_w13_mode<MOE_FP8_E4M3>(max_tiles, bb, ww, w13_scale, sorted_ids, tiles,
                                        num_tiles, H, I, k, act_amax_bits, h, amax_h_bits, st);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_w2_tiles(int mode, const void* b, const void* w2, const float* w2_scale,
                           const Tile* tiles, const int32_t* num_tiles, int max_tiles, int H,
                           int I, const uint32_t* act_amax_bits, float* y, hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  const char* bb = reinterpret_cast<const char*>(b);
  const char* ww = reinterpret_cast<const char*>(w2);
  if (mode == MOE_BF16)
    launch_tiles_w2_mode<MOE_BF16>(max_tiles, bb, ww, w2_scale, tiles, num_tiles, H, I,
                                   act_amax_bits, y, st);
  else if (mode == MOE_FP8_E4M3)
    launch_tiles_w2_mode<MOE_FP8_E4M3>(max_tiles, bb, ww, w2_scale, tiles, num_tiles, H, I,
                                       act_amax_bits, y, st);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
