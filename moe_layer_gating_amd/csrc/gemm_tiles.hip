// gemm_tiles.hip -- grouped expert GEMMs for many tokens per expert (prefill
// and mixed batches), FP8 e4m3 or bf16.
//
// When an expert receives tens to thousands of tokens, its weight rows are
// used against many tokens and the GEMM becomes a 2-D tiled contraction.  A
// block owns a 128*WN (weight rows) x BM (sorted positions of one expert)
// output tile and walks the reduction dimension K in 128-byte stages (128 FP8
// codes or 64 bf16 values per row).  Each of its 4*WN waves owns 32 weight
// rows (two 16-row MFMA tiles) and all BM columns.  With WN = 2 each staged
// token tile serves 256 weight rows, which halves the token-side L2 requests
// per weight byte (both operands' requests share the CU's path to L2).
//
// The expert rows sit on the MFMA row side and the tokens on the column side,
// as in the decode kernels (codebridge-ai.com, "aws-moe-kernel-wgmma-triton-
// ttft", section "1. Matrix swap"), and the dequantisation scales are applied
// to the fp32 accumulators in the epilogue (agentic-affairs.com, "Triton
// improves the FP8 execution path").
//
// Weights are streamed from HBM into registers with full-line loads (lane l
// of load i reads 16-byte chunk l % 8 of the wave's row 8i + l / 8, so each
// load instruction covers eight whole 128-byte lines), prefetched kPD stages
// ahead through a ring of kPD + 1 register slots per wave.  The MFMA operand
// layout wants 16 rows x 32 bytes per instruction instead (four lanes per
// row): loaded that way, every instruction touches 16 half-used lines, and
// L2-resident data then reached the CUs at a third of the full-line rate
// (9.8 against 30.9 TB/s, measured).  So each stage passes through a
// wave-private 4 KB LDS region: the ring slot is stored with the full-line
// lane layout and read back in MFMA layout, chunk c of wave row r kept at
// slot c ^ swz(r) like the token tile below, so neither the stores nor the
// fragment reads (16 rows at one chunk index) conflict in the LDS banks
// (counters: 51 M conflict cycles per gate/up launch with slot
// c ^ ((r >> 1) & 7), none with swz).  The
// MFMA operands and sums are those of the direct loads (bit-identical
// results).  The token tile is shared by the block's waves: it is prefetched
// into registers the same way and written to one of four LDS stage buffers
// two stages before use, with one barrier per two stages.  Tiles holding at
// most a quarter or a half of BM positions run a narrower copy of the main
// loop.
//
// LDS layout of a token stage: row r keeps its 16-byte chunk c at slot
// c ^ swz(r), swz(r) = (r ^ (r >> 3)) & 7.  Eight consecutive rows read at
// one chunk index then hit eight different slots, as do sixteen consecutive
// rows counted over two 128-byte bank rows, so neither the stores nor the
// MFMA fragment reads conflict in the LDS banks.
//
// In FP8 mode both projections run on the FP8 MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4, unit block scales): the many-token
// layers are bound by MFMA issue as much as by HBM, and the FP8 instruction
// does a 128-deep step in one issue where the bf16 one needs four.  Its
// fp32 sums carry the instruction's own rounding.
//
// Launch order: block b takes tile b / NB and weight-row block b % NB, with
// NB = (rows of the weight matrix) / (128*WN).  Blocks are dealt to the 8 XCDs
// round-robin, so when NB is a multiple of 8 a given weight-row block of an
// expert always runs on the same XCD and its reuse across the expert's
// token tiles can be served by that XCD's L2.  The 64-position down
// projection (experts of mostly one tile) instead gives XCD x the tiles
// [x n / 8, (x + 1) n / 8), each with all its row blocks: a tile's token rows
// are then fetched into one L2 instead of eight (the mixed layer's down
// projection ran 3.6-6% faster; with the 128-position tiles of the prefill
// layers such orders were slower).  The 128-position down projection of a
// Zipf-skewed prefill batch takes its tiles in the spread order the grouping
// writes (full tiles evenly among the partial ones); the kernels only
// follow the list they are given.
#include "moe_common.h"

namespace moe {

constexpr int kTileN = 128;  // weight rows per 4 waves
constexpr int kStageB = 128;  // bytes of K per row per stage
constexpr int kPD = 3;        // weight stages in flight per wave
constexpr int kTokBufs = 4;   // LDS token-chunk buffers (stages)
constexpr int kXcds = 8;      // block b is dispatched to XCD b % 8

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// One 128-byte K stage of a 16x16 output tile: each lane supplies 32 bytes
// of its row of each operand, as two 16-byte chunks (h = 0, 1).
template <int MODE>
struct TileMma;

// FP8: one v_mfma_scale_f32_16x16x128_f8f6f4 over chunks 2g and 2g+1.
template <>
struct TileMma<MOE_FP8_E4M3> {
  static __device__ __forceinline__ int chunk(int g, int h) { return 2 * g + h; }
  static __device__ __forceinline__ f32x4 mma(i32x8 a, i32x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// bf16: two v_mfma_f32_16x16x32_bf16, the first over chunk g, the second
// over chunk 4+g.
template <>
struct TileMma<MOE_BF16> {
  static __device__ __forceinline__ int chunk(int g, int h) { return 4 * h + g; }
  static __device__ __forceinline__ f32x4 mma(i32x8 a, i32x8 b, f32x4 c) {
    i32x4 a0 = {a[0], a[1], a[2], a[3]}, a1 = {a[4], a[5], a[6], a[7]};
    i32x4 b0 = {b[0], b[1], b[2], b[3]}, b1 = {b[4], b[5], b[6], b[7]};
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0),
                                                __builtin_bit_cast(bf16x8, b0), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1),
                                                   __builtin_bit_cast(bf16x8, b1), c, 0, 0, 0);
  }
};

__device__ __forceinline__ i32x8 join(i32x4 lo, i32x4 hi) {
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Main loop shared by both projections.
//   a_rows[i]: this lane's weight row of full-line load i, at its chunk
//              (K offset 0);
//   b_rows[i]: this thread's staged token rows r0 + 32*WN*i, already offset
//              by the thread's chunk (t & 7) * 16;
//   acc[i][j]: row tile i, column tile j of the wave's 32 x BM accumulator.
// LDS bytes of one token-stage buffer.
template <int MODE, int BM>
constexpr int stage_lds_bytes() {
  return BM * kStageB;
}

template <int MODE, int BM, int WN, int PD, int MTA>
__device__ __forceinline__ void tile_mainloop(const char* const* a_rows, const char* const* b_rows,
                                              int n_stages, char* lds, f32x4 (*acc)[MTA]) {
  static_assert(BM / 16 <= MTA && (BM % (32 * WN) == 0 || BM == 16 * WN), "tile shape");
  typedef TileMma<MODE> M;
  constexpr int ROWB = kStageB;  // LDS bytes per token row
  constexpr int B_BYTES = stage_lds_bytes<MODE, BM>();
  // token rows staged per thread; a stage of fewer than 32*WN rows is staged
  // by the threads with r0 < BM only (whole waves)
  constexpr int NB = BM >= 32 * WN ? BM / (32 * WN) : 1;
  constexpr bool ALL_STAGE = BM >= 32 * WN;
  constexpr int MT = BM / 16;            // column tiles
  const int t = threadIdx.x;
  const int lane = lane_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int c = t & 7, r0 = t >> 3;

  int b_slot[NB];
#pragma unroll
  for (int i = 0; i < NB; i++) {
    const int r = r0 + 32 * WN * i;
    b_slot[i] = r * ROWB + ((c ^ swz(r)) << 4);
  }
  auto stage_b = [&](char* buf, const i32x4* src) {
    if (!ALL_STAGE && r0 >= BM) return;
#pragma unroll
    for (int i = 0; i < NB; i++) *reinterpret_cast<i32x4*>(buf + b_slot[i]) = src[i];
  };
  // LDS offsets of this lane's two chunks in column tile j: row j*16 + r16,
  // whose swizzle is (r16 ^ (2j + r16 / 8)) & 7.
  const int b_base = r16 * ROWB;
  const int cb0 = M::chunk(g, 0), cb1 = M::chunk(g, 1), r16h = r16 >> 3;
  // the wave's weight stage in LDS: 32 rows of 128 B, chunk c of wave row r
  // at slot c ^ swz(r); written from the full-line loads (lane l:
  // row 8i + l / 8, chunk l % 8 of load i), read back in MFMA layout
  char* wbuf = lds + kTokBufs * B_BYTES + (t / kWave) * 4096;
  int w_st[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int r = 8 * i + (lane >> 3), cc = lane & 7;
    w_st[i] = r * 128 + ((cc ^ swz(r)) << 4);
  }
  int w_ld[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int r = 16 * i + r16;
    w_ld[i][0] = r * 128 + ((cb0 ^ swz(r)) << 4);
    w_ld[i][1] = r * 128 + ((cb1 ^ swz(r)) << 4);
  }

  // Weights are prefetched PD stages ahead, token chunks PD + 1 stages ahead,
  // both through rings of PD + 1 register slots, and the loads of a stage go
  // out before its MFMAs.  A token chunk is written to LDS two stages before
  // use, into one of kTokBufs = 4 stage buffers, so one barrier per two
  // stages both publishes the next two chunks and retires the two buffers
  // just read (a barrier per stage cost 6-12% of the gate/up time).  A wave's
  // loads complete in issue order, so each stage issues its token chunk
  // before its weights: the wait for chunk s+2 at stage s then covers the
  // weights of stage s only, never those of s+1.  Prefetch stage indices are
  // clamped to the last stage (an overrun re-reads it), and the stages that
  // pad the final group of PD + 1 skip their MFMAs by a block-uniform branch
  // (fewer VGPRs than zero weight fragments, and 1.5-2% faster).
  static_assert(PD == 3 && kTokBufs == 4, "prologue and ring written for PD = 3");
  const int last = n_stages - 1;
  auto load_a = [&](int kt, i32x4* dst) {
    const size_t off = (size_t)kt * kStageB;
#pragma unroll
    for (int i = 0; i < 4; i++) dst[i] = *reinterpret_cast<const i32x4*>(a_rows[i] + off);
  };
  auto load_b = [&](int kt, i32x4* dst) {
    if (!ALL_STAGE && r0 >= BM) return;
    const size_t off = (size_t)kt * kStageB;
#pragma unroll
    for (int i = 0; i < NB; i++) dst[i] = *reinterpret_cast<const i32x4*>(b_rows[i] + off);
  };
  constexpr int RING = PD + 1;
  i32x4 ra[RING][4];   // weights of stage s in slot s % RING
  i32x4 rb[RING][NB];  // token chunk of stage s in slot s % RING
  // chunks of stages 0-3 and weights of stages 0-2, chunk before weights
  load_b(0, rb[0]);
  load_b(min(1, last), rb[1]);
  load_a(0, ra[0]);
  load_b(min(2, last), rb[2]);
  load_a(min(1, last), ra[1]);
  load_b(min(3, last), rb[3]);
  load_a(min(2, last), ra[2]);
  stage_b(lds, rb[0]);
  stage_b(lds + B_BYTES, rb[1]);
  __syncthreads();

  const int n_groups = (n_stages + RING - 1) / RING;
  for (int grp = 0; grp < n_groups; grp++) {
#pragma unroll
    for (int q = 0; q < RING; q++) {
      const int kt = grp * RING + q;
      // slot q held the chunk of stage kt, written to LDS two stages ago
      load_b(min(kt + RING, last), rb[q]);
      load_a(min(kt + PD, last), ra[(q + PD) % RING]);
      // keeps this stage's MFMAs and the consumers of the stages in flight
      // from being scheduled up against the loads just issued (measured: FP8
      // down projection 1.5% faster)
      __builtin_amdgcn_sched_barrier(0);
      const bool valid = kt < n_stages;
      // weights of this stage through the wave's LDS region into MFMA layout
#pragma unroll
      for (int i = 0; i < 4; i++) *reinterpret_cast<i32x4*>(wbuf + w_st[i]) = ra[q][i];
      i32x8 af[2];
#pragma unroll
      for (int i = 0; i < 2; i++)
        af[i] = join(*reinterpret_cast<const i32x4*>(wbuf + w_ld[i][0]),
                     *reinterpret_cast<const i32x4*>(wbuf + w_ld[i][1]));
      const i32x8 a0 = af[0], a1 = af[1];
      const char* cur = lds + q * B_BYTES;
      // the wave's priority is raised over its MFMA burst (16k-token FP8
      // down projection 2% faster)
      __builtin_amdgcn_s_setprio(1);
      if (valid) {  // block-uniform: the stages that pad the final group skip
#pragma unroll
        for (int j = 0; j < MT; j++) {
          const int sw = (r16 ^ (2 * j + r16h)) & 7;
          const char* rowp = cur + j * 16 * kStageB + b_base;
          const i32x8 fb = join(*reinterpret_cast<const i32x4*>(rowp + ((cb0 ^ sw) << 4)),
                                *reinterpret_cast<const i32x4*>(rowp + ((cb1 ^ sw) << 4)));
          acc[0][j] = M::mma(a0, fb, acc[0][j]);
          acc[1][j] = M::mma(a1, fb, acc[1][j]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // the token chunk of stage kt+2 into its LDS buffer, last read at
      // stage kt-2 (before the previous barrier)
      __builtin_amdgcn_sched_barrier(0);
      stage_b(lds + ((q + 2) % RING) * B_BYTES, rb[(q + 2) % RING]);
      if (q & 1) __syncthreads();
    }
  }
}

// A tile holding at most a quarter or a half of BM positions runs the main
// loop over BM / 4 or BM / 2 columns only (a block-uniform choice between
// fully unrolled loops): Zipf-routed prefill tiles are 46% full on average,
// and the MFMAs, LDS reads and token loads of the all-padding columns are
// skipped.
template <int MODE, int BM, int WN, int PD>
__device__ __forceinline__ void run_mainloop(int mt, const char* const* a_rows,
                                             const char* const* b_rows, int n_stages, char* lds,
                                             f32x4 (*acc)[BM / 16]) {
  if constexpr (BM == 128) {
    if (mt <= BM / 4) {
      tile_mainloop<MODE, BM / 4, WN, PD, BM / 16>(a_rows, b_rows, n_stages, lds, acc);
      return;
    }
  }
  if constexpr (BM / 2 >= 32 * WN || BM / 2 == 16 * WN) {
    if (mt <= BM / 2) {
      tile_mainloop<MODE, BM / 2, WN, PD, BM / 16>(a_rows, b_rows, n_stages, lds, acc);
      return;
    }
  }
  tile_mainloop<MODE, BM, WN, PD, BM / 16>(a_rows, b_rows, n_stages, lds, acc);
}

// ------------------------------------------------------------------- w13
// Block row R (wave R / 32, row tile (R / 16) % 2, MFMA row R % 16): tile
// q = R / 16 row 2i is gate feature F + 8q + i (F = nb*64*WN), row 2i+1 the
// matching up feature, so a lane's accumulator rows 4g..4g+3 hold
// gate/up/gate/up of features F + 8q + 2g and + 1.
template <int MODE, int BM, int WN, int PD = kPD>
__global__ __launch_bounds__(256 * WN)
__attribute__((amdgpu_waves_per_eu(2, 2))) void w13_swiglu_tiles(
    const char* __restrict__ b, const char* __restrict__ w13, const float* __restrict__ w13_scale,
    const int32_t* __restrict__ sorted_ids, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, int H, int I, int k, const uint32_t* act_amax_bits,
    void* __restrict__ h, uint32_t* amax_h_bits) {
  constexpr int ES = MODE == MOE_BF16 ? 2 : 1;
  constexpr int MT = BM / 16;
  __shared__ __attribute__((aligned(16))) char lds[kTokBufs * stage_lds_bytes<MODE, BM>() +
                                                    4096 * 4 * WN];
  const int NBLK = 2 * I / (kTileN * WN);
  const int tile_idx = blockIdx.x / NBLK;
  const int nb = blockIdx.x - tile_idx * NBLK;
  if (tile_idx >= *num_tiles) return;
  const Tile tl = tiles[tile_idx];
  const int t = threadIdx.x, c = t & 7, r0 = t >> 3;
  const int lane = lane_id(), w = t / kWave;
  const int r16 = lane & 15, g = lane >> 4;
  const size_t row_bytes = (size_t)H * ES;

  // full-line weight loads: load i of lane l reads chunk l % 8 of the
  // wave's row 8i + l / 8, i.e. MFMA row tile wr / 16, row wr % 16
  const char* a_rows[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int wr = 8 * i + (lane >> 3), rr = wr & 15;
    const int q = 2 * w + (wr >> 4);
    const int f = nb * 64 * WN + q * 8 + (rr >> 1);
    const int wrow = (rr & 1) ? I + f : f;
    a_rows[i] = w13 + ((size_t)tl.e * 2 * I + wrow) * row_bytes + (lane & 7) * 16;
  }
  const char* b_rows[BM / (32 * WN)];
#pragma unroll
  for (int i = 0; i < BM / (32 * WN); i++) {
    const int j = min(r0 + 32 * WN * i, tl.mt - 1);
    const int tok = sorted_ids[tl.p0 + j] / k;
    b_rows[i] = b + (size_t)tok * row_bytes + c * 16;
  }
  f32x4 acc[2][MT];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < MT; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  run_mainloop<MODE, BM, WN, PD>(tl.mt, a_rows, b_rows, (int)(row_bytes / kStageB), lds, acc);

  float cs = 1.0f;
  if (is_fp8(MODE)) {
    const float a = __uint_as_float(*act_amax_bits);
    cs = (a > 0.f ? a / 448.0f : 1.0f) * w13_scale[tl.e];
  }
  float hmax = 0.f;
#pragma unroll
  for (int j = 0; j < MT; j++) {
    const int col = j * 16 + r16;
    if (col < tl.mt) {
      uint16_t* hrow = reinterpret_cast<uint16_t*>(h) + (size_t)(tl.p0 + col) * I;
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const int f = nb * 64 * WN + (2 * w + i) * 8 + 2 * g;
        float hv[2];
#pragma unroll
        for (int q = 0; q < 2; q++) {
          float gv = acc[i][j][2 * q], uv = acc[i][j][2 * q + 1];
          if (is_fp8(MODE)) {
            gv *= cs;
            uv *= cs;
          }
          hv[q] = gv / (1.0f + expf(-gv)) * uv;
        }
        const uint16_t h0 = f32_to_bf16(hv[0]), h1 = f32_to_bf16(hv[1]);
        *reinterpret_cast<uint32_t*>(hrow + f) = (uint32_t)h0 | ((uint32_t)h1 << 16);
        hmax = fmaxf(hmax, fmaxf(fabsf(bf16_to_f32(h0)), fabsf(bf16_to_f32(h1))));
      }
    }
  }
  if (is_fp8(MODE)) {
    hmax = wave_max(hmax);
    if (lane == 0) {
      const uint32_t bits = __float_as_uint(hmax);
      if (bits > __atomic_load_n(amax_h_bits, __ATOMIC_RELAXED)) atomicMax(amax_h_bits, bits);
    }
  }
}

// -------------------------------------------------------------------- w2
// YB: y is stored in bf16 (the FP8 fused path; the scaled fp32 accumulators
// rounded to nearest even), else in fp32.
template <int MODE, int BM, int WN, bool YB, int PD = kPD>
__global__ __launch_bounds__(256 * WN)
__attribute__((amdgpu_waves_per_eu(2, 2))) void w2_tiles(const char* __restrict__ b,
                                                const char* __restrict__ w2,
                                                const float* __restrict__ w2_scale,
                                                const Tile* __restrict__ tiles,
                                                const int32_t* __restrict__ num_tiles, int H, int I,
                                                const uint32_t* act_amax_bits,
                                                void* __restrict__ y) {
  constexpr int ES = MODE == MOE_FP8_E4M3 ? 1 : 2;
  constexpr int MT = BM / 16;
  __shared__ __attribute__((aligned(16))) char lds[kTokBufs * BM * kStageB + 4096 * 4 * WN];
  const int NBLK = H / (kTileN * WN);
  int tile_idx, nb;
  if constexpr (BM == 64) {
    // XCD x = b % 8 takes tiles [x n / 8, (x + 1) n / 8), tile by tile
    const int n = *num_tiles, x = blockIdx.x % kXcds, s = blockIdx.x / kXcds;
    const int lo = (int)((long)x * n / kXcds), hi = (int)((long)(x + 1) * n / kXcds);
    if (s >= (hi - lo) * NBLK) return;
    tile_idx = lo + s / NBLK;
    nb = s - (tile_idx - lo) * NBLK;
  } else {
    tile_idx = blockIdx.x / NBLK;
    nb = blockIdx.x - tile_idx * NBLK;
    if (tile_idx >= *num_tiles) return;
  }
  const Tile tl = tiles[tile_idx];
  const int t = threadIdx.x, c = t & 7, r0 = t >> 3;
  const int lane = lane_id(), w = t / kWave;
  const int r16 = lane & 15, g = lane >> 4;
  const size_t row_bytes = (size_t)I * ES;

  const char* a_rows[4];
#pragma unroll
  for (int i = 0; i < 4; i++)
    a_rows[i] = w2 + ((size_t)tl.e * H + nb * kTileN * WN + w * 32 + 8 * i + (lane >> 3)) *
                         row_bytes + (lane & 7) * 16;
  const char* b_rows[BM / (32 * WN)];
#pragma unroll
  for (int i = 0; i < BM / (32 * WN); i++) {
    const int j = min(r0 + 32 * WN * i, tl.mt - 1);
    b_rows[i] = b + (size_t)(tl.p0 + j) * row_bytes + c * 16;
  }
  f32x4 acc[2][MT];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < MT; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  run_mainloop<MODE, BM, WN, PD>(tl.mt, a_rows, b_rows, (int)(row_bytes / kStageB), lds, acc);

  float cs = 1.0f;
  if (MODE == MOE_FP8_E4M3) {
    const float a = __uint_as_float(*act_amax_bits);
    cs = (a > 0.f ? a / 448.0f : 1.0f) * w2_scale[tl.e];
  }
#pragma unroll
  for (int j = 0; j < MT; j++) {
    const int col = j * 16 + r16;
    if (col < tl.mt) {
      const size_t yo = (size_t)(tl.p0 + col) * H + nb * kTileN * WN + w * 32;
#pragma unroll
      for (int i = 0; i < 2; i++) {
        f32x4 v = acc[i][j];
        if (MODE == MOE_FP8_E4M3) v *= cs;
        const size_t o = yo + i * 16 + 4 * g;
        if (YB) {
          const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + o) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(y) + o) = v;
        }
      }
    }
  }
}

// 8-wave blocks (256 weight rows) where the row count allows: always for
// the gate/up projection, and for the down projection with 128-position
// tiles only; else 4-wave blocks.  Measured: with 8 waves the prefill down
// projection ran 4% faster and the mixed layer's 64-position gate/up 3%
// faster, while the mixed layer's 64-position down projection ran 8% slower.
inline int tiles_wn(bool gate_up, int bm, long rows) {
  return ((gate_up || bm == 128) && rows % (2 * kTileN) == 0) ? 2 : 1;
}

template <int MODE, int BM>
static void launch_tiles_w13_mode(long max_tiles, const char* b, const char* w13,
                                  const float* w13_scale, const int32_t* sorted_ids,
                                  const Tile* tiles, const int32_t* num_tiles, int H, int I, int k,
                                  const uint32_t* act_amax_bits, void* h, uint32_t* amax_h_bits,
                                  hipEvent_t e0, hipEvent_t e1, hipStream_t st) {
  if (tiles_wn(true, BM, 2L * I) == 2)
    launch_on(w13_swiglu_tiles<MODE, BM, 2>, dim3(max_tiles * (2L * I / (2 * kTileN))),
              dim3(512), st, e0, e1, b, w13, w13_scale, sorted_ids, tiles, num_tiles, H, I, k,
              act_amax_bits, h, amax_h_bits);
  else
    launch_on(w13_swiglu_tiles<MODE, BM, 1>, dim3(max_tiles * (2L * I / kTileN)), dim3(256), st,
              e0, e1, b, w13, w13_scale, sorted_ids, tiles, num_tiles, H, I, k, act_amax_bits, h,
              amax_h_bits);
}

template <int MODE, int BM, bool YB>
static void launch_tiles_w2_mode(long max_tiles, const char* b, const char* w2,
                                 const float* w2_scale, const Tile* tiles,
                                 const int32_t* num_tiles, int H, int I,
                                 const uint32_t* act_amax_bits, void* y, hipEvent_t e0,
                                 hipEvent_t e1, hipStream_t st) {
  // the 64-position order gives each XCD up to ceil(max_tiles / 8) tiles
  if (BM == 64) max_tiles = (max_tiles + kXcds - 1) / kXcds * kXcds;
  if (tiles_wn(false, BM, H) == 2)
    launch_on(w2_tiles<MODE, BM, 2, YB>, dim3(max_tiles * (long)(H / (2 * kTileN))), dim3(512),
              st, e0, e1, b, w2, w2_scale, tiles, num_tiles, H, I, act_amax_bits, y);
  else
    launch_on(w2_tiles<MODE, BM, 1, YB>, dim3(max_tiles * (long)(H / kTileN)), dim3(256), st, e0,
              e1, b, w2, w2_scale, tiles, num_tiles, H, I, act_amax_bits, y);
}

hipError_t launch_w13_tiles(int mode, int bm, const void* b, const void* w13,
                            const float* w13_scale, const int32_t* sorted_ids, const Tile* tiles,
                            const int32_t* num_tiles, int max_tiles, int H, int I, int k,
                            const uint32_t* act_amax_bits, void* h, uint32_t* amax_h_bits,
                            hipEvent_t e0, hipEvent_t e1, hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  const char* bb = reinterpret_cast<const char*>(b);
  const char* ww = reinterpret_cast<const char*>(w13);
#define MOE_W13_TILES(MODE_, BM_)                                                             \
  launch_tiles_w13_mode<MODE_, BM_>(max_tiles, bb, ww, w13_scale, sorted_ids, tiles, num_tiles, \
                                    H, I, k, act_amax_bits, h, amax_h_bits, e0, e1, st)
  if (mode == MOE_BF16 && bm == 64)
    MOE_W13_TILES(MOE_BF16, 64);
  else if (mode == MOE_BF16 && bm == 128)
    MOE_W13_TILES(MOE_BF16, 128);
  else if (mode == MOE_FP8_E4M3 && bm == 64)
    MOE_W13_TILES(MOE_FP8_E4M3, 64);
  else if (mode == MOE_FP8_E4M3 && bm == 128)
    MOE_W13_TILES(MOE_FP8_E4M3, 128);
  else
    return hipErrorInvalidValue;
#undef MOE_W13_TILES
  return hipGetLastError();
}

hipError_t launch_w2_tiles(int mode, int bm, const void* b, const void* w2, const float* w2_scale,
                           const Tile* tiles, const int32_t* num_tiles, int max_tiles, int H,
                           int I, const uint32_t* act_amax_bits, void* y, bool y_bf16,
                           hipEvent_t e0, hipEvent_t e1, hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  const char* bb = reinterpret_cast<const char*>(b);
  const char* ww = reinterpret_cast<const char*>(w2);
#define MOE_W2_TILES(MODE_, BM_, YB_)                                                           \
  launch_tiles_w2_mode<MODE_, BM_, YB_>(max_tiles, bb, ww, w2_scale, tiles, num_tiles, H, I,    \
                                        act_amax_bits, y, e0, e1, st)
  if (y_bf16 && mode != MOE_FP8_E4M3) return hipErrorInvalidValue;
  if (mode == MOE_BF16 && bm == 64)
    MOE_W2_TILES(MOE_BF16, 64, false);
  else if (mode == MOE_BF16 && bm == 128)
    MOE_W2_TILES(MOE_BF16, 128, false);
  else if (mode == MOE_FP8_E4M3 && bm == 64 && !y_bf16)
    MOE_W2_TILES(MOE_FP8_E4M3, 64, false);
  else if (mode == MOE_FP8_E4M3 && bm == 128 && !y_bf16)
    MOE_W2_TILES(MOE_FP8_E4M3, 128, false);
  else if (mode == MOE_FP8_E4M3 && bm == 64)
    MOE_W2_TILES(MOE_FP8_E4M3, 64, true);
  else if (mode == MOE_FP8_E4M3 && bm == 128)
    MOE_W2_TILES(MOE_FP8_E4M3, 128, true);
  else
    return hipErrorInvalidValue;
#undef MOE_W2_TILES
  return hipGetLastError();
}

}  // namespace moe
