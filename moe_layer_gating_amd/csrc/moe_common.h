// moe_common.h -- device helpers and internal launcher declarations shared by
// the HIP translation units of the fused MoE library (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_gfx950.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kSkinnyBM = 16;  // sorted positions per tile of the few-token GEMMs
constexpr int kRouteSmallMax = 256;  // pairs routed by the one-block front kernel
// x values the one-block front kernel quantises in its second block; a larger
// x goes to the grid-wide amax and quantisation passes (one block streams
// about 0.1 TB/s, the grid-wide passes the whole chip's bandwidth)
constexpr long kFrontQuantMax = 131072;
constexpr int kSortChunk = 1024;     // pairs per chunk of the many-pair grouping (one per thread)
constexpr int kChunkSortMin = 8192;  // pairs from which the chunked grouping is used
constexpr int kTilesBMMin = 64;  // smallest tile of the many-token GEMMs (64 or 128 positions)
constexpr int kRouterBM = 64;    // tokens per tile of the tiled router GEMM
constexpr int kFusedRouterMaxTE = 4096;  // logits the front kernel keeps in LDS (T * E)
// router weights (E * H bf16 values) the front kernel reads itself: one CU
// streams them, so beyond this a separate many-block router launch is faster
// (measured: E = 64, H = 4096 cost 15 us in one block against 10 us for the
// separate launch)
constexpr long kFusedRouterMaxEH = 131072;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Internal kernel operand mode: FP8 e4m3 codes widened to bf16 in registers
// and multiplied on the bf16 MFMA.  Every e4m3 value is exact in bf16 and the
// bf16 MFMA sums these products in fp32 (bit-equal to the rounded exact sum
// 99% of the time, measured); the FP8 MFMA keeps fewer bits (about 2^-19 of
// sum|p| per instruction, measured), and its error flips rounding decisions
// made on the result (about 2% of h's bf16 values).  Used for the gate/up
// projection of the few-token kernels, which stream weights from HBM: there
// the four bf16 MFMAs per 128-code step were measured as fast as one FP8
// MFMA.  The many-token tiled kernels, bound by MFMA issue, take the FP8
// MFMA for both projections.
constexpr int kFp8ViaBf16 = 3;
__host__ __device__ constexpr bool is_fp8(int mode) {
  return mode == MOE_FP8_E4M3 || mode == kFp8ViaBf16;
}

// Eight e4m3 codes (little-endian in lo, hi) as eight bf16 values, exactly.
__device__ __forceinline__ i32x4 e4m3x8_to_bf16x8(int lo, int hi) {
  return i32x4{__builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
               __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
               __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
               __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
}

// One unit of grouped-GEMM work: `mt` consecutive sorted positions starting
// at `p0`, all routed to expert `e`.
struct Tile {
  int32_t e, p0, mt, pad;
};

// Control words at the start of the workspace (zeroed at the start of a call
// by the first kernel that runs).
struct Ctrl {
  uint32_t amax_x_bits;    // max |x| as fp32 bits (non-negative floats order as uints)
  uint32_t amax_h_bits;    // max |h| as fp32 bits
  int32_t num_tiles;       // tiles of <= kSkinnyBM positions written by the tile builder
  int32_t num_tiles_big;   // tiles of the many-token GEMMs
  int32_t num_tiles_router;  // token tiles of the tiled router GEMM
  int32_t pad[59];
};
static_assert(sizeof(Ctrl) == 256, "ctrl block is one 256-byte slot");

// ----------------------------------------------------------------- numerics
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Eight bf16 values times r as eight OCP e4m3fn codes (element i in byte i):
// fl32(v * r), rounded to nearest even and saturated to +-448 (subnormals
// kept).  gfx950's v_cvt_pk_fp8_f32 rounds to nearest even in the OCP format;
// the clamp to +-448 in front of it makes it saturate, and with it the
// conversion was checked equal, on every non-NaN fp32 input, to a software
// encoder written from the format's definition (drop 20 fraction bits with a
// nearest-even carry and rebias 127 -> 7; below 2^-6, round v * 2^9 to an
// integer).  NaN inputs are outside the contract (x and h hold no NaN).
__device__ __forceinline__ uint2 bf16x8_to_e4m3x8(i32x4 v, float r) {
  float f[8];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const uint32_t u = (uint32_t)v[q];
    f[2 * q] = __builtin_amdgcn_fmed3f(bf16_to_f32((uint16_t)(u & 0xffffu)) * r, -448.0f, 448.0f);
    f[2 * q + 1] = __builtin_amdgcn_fmed3f(bf16_to_f32((uint16_t)(u >> 16)) * r, -448.0f, 448.0f);
  }
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// ----------------------------------------------------------------- wave ops
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Launch `kern` on `st`; when e0 / e1 are given they take the kernel's own
// start / end time (hipExtLaunchKernelGGL), which is how the stage-timing
// entry point times the GEMMs without marker packets around them.
template <typename... KArgs, typename... Args>
inline void launch_on(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t st, hipEvent_t e0,
                      hipEvent_t e1, Args... args) {
  if (e0 || e1)
    hipExtLaunchKernelGGL(kern, grid, block, 0, st, e0, e1, 0, static_cast<KArgs>(args)...);
  else
    kern<<<grid, block, 0, st>>>(static_cast<KArgs>(args)...);
}

// FP8 quantisation of x carried by extra blocks of the gating and grouping
// launches of the many-pair path, next to their latency-bound work: the
// gating launch's extra blocks each write the max |x| of their slice to
// part[b] (no atomics, so nothing waits for the zeroed control block); the
// grouping launch's extra blocks each reduce the kXParts partials, the first
// writes amax(x) to ctrl->amax_x_bits, and all encode their slice of x.
constexpr int kXParts = 256;    // partial-max blocks
constexpr int kXQuantBlocks = 256;  // encoding blocks
struct XWork {
  const uint16_t* x;  // bf16, 8 * n8 values, 16-byte aligned
  long n8;
  float* part;        // kXParts floats of workspace
  Ctrl* ctrl;
  uint8_t* xq;        // e4m3 codes
};

// --------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  All work goes to `st`.
// With xw, the gating launch also writes the partial maxima of |x| and the
// grouping launch (align sort or chunk sort) encodes x.
hipError_t launch_topk_gating(const float* logits, int T, int E, int k, int renorm, int32_t* ids,
                              float* w, uint32_t* zero_words, int n_zero, hipStream_t st,
                              const XWork* xw = nullptr);
hipError_t launch_align_sort(const int32_t* ids, int T, int k, int E, int32_t* counts,
                             int32_t* offsets, int32_t* sorted_ids, int32_t* inv_perm,
                             hipStream_t st, const XWork* xw = nullptr);
// Gating, grouping, tile list and (xq != nullptr) FP8 quantisation of x in
// one block, for T*k <= kRouteSmallMax; inv_perm may be null.  With wg (bf16
// router weights [E,H], T*E <= kFusedRouterMaxTE) the logits are computed in
// the kernel from x and wg (and copied to logits_out if that is given);
// otherwise they are read from `logits`.  With neither, the ids are read from
// `ids` and only the grouping and the tile list are formed.  The tile count
// goes to ctrl->num_tiles_big when `big`, else to ctrl->num_tiles.  Writes
// every control word.
hipError_t launch_route_small(const float* logits, int T, int E, int k, int renorm, int32_t* ids,
                              float* w, int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                              int32_t* inv_perm, int bm, bool big, Tile* tiles, Ctrl* ctrl,
                              const uint16_t* x, int H, uint8_t* xq, const uint16_t* wg,
                              float* logits_out, hipStream_t st);
// Grouping of n pairs in chunks of kSortChunk plus the tile list of <= bm
// positions (three launches).  Scratch: chunk_counts and base hold
// ceil(n / kSortChunk) * E ints each, rank n ints.
// With tiles_spread, the chunked grouping also writes the tile list in the
// down projection's launch order (full tiles spread evenly among the others).
hipError_t launch_chunk_sort(const int32_t* ids, int n, int E, int32_t* counts, int32_t* offsets,
                             int32_t* sorted_ids, int32_t* inv_perm, int bm, Tile* tiles,
                             int32_t* num_tiles, int32_t* chunk_counts, int32_t* base,
                             int32_t* rank, hipStream_t st, const XWork* xw = nullptr,
                             Tile* tiles_spread = nullptr);
hipError_t launch_build_tiles(const int32_t* offsets, int E, int bm, Tile* tiles,
                              int32_t* num_tiles, hipStream_t st);
hipError_t launch_zero_words(uint32_t* p, int n, hipStream_t st);
// Router GEMM logits[t][e] = x[t] . wg[e] (fp32 accumulation); `tiles` holds
// ceil(T / kRouterBM) entries and *num_tiles is written (tiled path only).
bool router_uses_tiles(int mode, int T, int E);
hipError_t launch_router_logits(int mode, const void* x, const void* wg, int T, int H, int E,
                                float* logits, Tile* tiles, int32_t* num_tiles, int max_tiles,
                                hipStream_t st);
hipError_t launch_amax_bf16(const uint16_t* src, long n, uint32_t* amax_bits, hipStream_t st);
hipError_t launch_quant_e4m3(const uint16_t* src, long n, const uint32_t* amax_bits, uint8_t* dst,
                             hipStream_t st);
hipError_t launch_write_scales(const Ctrl* ctrl, float* act_scales, hipStream_t st);
// scales[0] = amax / 448 (or 1) from the amax bits in scales[1].
hipError_t launch_finish_scale(float* scales, hipStream_t st);
// Grouped GEMMs.  `b` is the token-side operand: x (fp32/bf16) or the e4m3
// codes of x (FP8) for w13; h (fp32/bf16) or the codes of h (FP8) for w2.
// `act_amax_bits` (FP8 only) points at amax of that activation as fp32 bits.
hipError_t launch_w13_swiglu(int mode, const void* b, const void* w13, const float* w13_scale,
                             const int32_t* sorted_ids, const Tile* tiles, const Ctrl* ctrl,
                             int max_tiles, int H, int I, int k, const uint32_t* act_amax_bits,
                             void* h, uint32_t* amax_h_bits, hipEvent_t e0, hipEvent_t e1,
                             hipStream_t st);
hipError_t launch_w2(int mode, const void* b, const void* w2, const float* w2_scale,
                     const Tile* tiles, const Ctrl* ctrl, int max_tiles, int H, int I,
                     const uint32_t* act_amax_bits, float* y, hipEvent_t e0, hipEvent_t e1,
                     hipStream_t st);
// Many-token variants (bf16 and FP8 only; tiles of bm = 64 or 128 sorted
// positions); the tile count is read from *num_tiles on the device.
hipError_t launch_w13_tiles(int mode, int bm, const void* b, const void* w13,
                            const float* w13_scale, const int32_t* sorted_ids, const Tile* tiles,
                            const int32_t* num_tiles, int max_tiles, int H, int I, int k,
                            const uint32_t* act_amax_bits, void* h, uint32_t* amax_h_bits,
                            hipEvent_t e0, hipEvent_t e1, hipStream_t st);
// y_bf16 (FP8 only): y is stored in bf16 instead of fp32.
hipError_t launch_w2_tiles(int mode, int bm, const void* b, const void* w2, const float* w2_scale,
                           const Tile* tiles, const int32_t* num_tiles, int max_tiles, int H,
                           int I, const uint32_t* act_amax_bits, void* y, bool y_bf16,
                           hipEvent_t e0, hipEvent_t e1, hipStream_t st);
// Inverse rotary embedding + per-head e4m3 quantisation (rope.hip); shapes
// already checked by the caller (head_dim / 8 <= 64 lanes per head).
hipError_t launch_inv_rope_fp8(const uint16_t* x, const int32_t* positions, const float* cos_sin,
                               int T, int n_heads, int head_dim, int rot_dim, int max_pos,
                               bool interleaved, uint8_t* codes, float* scales, hipStream_t st);
// y [T*k,H] in sorted order, fp32 or (y_bf16, not in fp32 mode) bf16.
hipError_t launch_combine(int mode, const void* y, bool y_bf16, const int32_t* inv_perm,
                          const float* w, int T, int H, int k, void* out, hipStream_t st);

}  // namespace moe
