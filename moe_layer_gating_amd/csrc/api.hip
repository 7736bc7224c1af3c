// api.cpp -- host side of the fused MoE library: argument checks, workspace
// carve-up and the launch sequences behind the C ABI in include/moe_gfx950.h.
//
// Nothing here is specialised on the token count or on the per-expert
// counts: they are runtime values read by the kernels on the device, so a
// new batch size never triggers a rebuild (the lesson of codebridge-ai.com,
// "aws-moe-kernel-wgmma-triton-ttft", section "3. Kill JIT recompilation",
// applied to an ahead-of-time library).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "moe_common.h"

using namespace moe;

// Scratch of moe_fused_forward_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never passes `scratch`
// itself to a kernel (on the host it only names the symbol); it uses the
// device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int act_bytes(int wdtype) { return wdtype == MOE_F32 ? 4 : 2; }

inline int w_bytes(int wdtype) {
  return wdtype == MOE_F32 ? 4 : (wdtype == MOE_BF16 ? 2 : 1);
}

inline long max_tiles_for(long n_pairs, int E, int bm) {
  long nz = n_pairs < E ? n_pairs : E;  // experts that can be non-empty
  return n_pairs / bm + nz;
}

// Offsets of the workspace regions for one shape.
struct Layout {
  size_t ctrl, ids, wts, counts, offsets, sorted, inv, tiles, tiles_big, tiles_spread,
      chunk_counts, chunk_base,
      rank, xpart, xq, hq, h, y, logits, rtiles, total;
  long max_tiles, max_tiles_big, max_rtiles;
};

// Shape class: the many-token tiled GEMMs once experts receive 16 or more
// pairs on average (bf16 and FP8); the few-token swap-AB GEMMs otherwise.
// The tiled GEMMs use 64-position tiles while the mean is below 64 pairs
// per expert (less padding), 128-position tiles above (more weight reuse).
// Decided from the shape alone, so no per-call specialisation arises.
inline bool use_tiles(const moe_shape& s) {
  return s.wdtype != MOE_F32 && (long)s.T * s.k >= 16L * s.E;
}
inline int tiles_bm(const moe_shape& s) { return (long)s.T * s.k < 64L * s.E ? 64 : 128; }

// Grouping kernels by pair count, the same for the fused entry point and for
// moe_align_sort: one block (gating or given ids, grouping, the tile list, and
// in the fused FP8 call the x quantisation) up to kRouteSmallMax pairs; one
// block per expert below kChunkSortMin pairs; the chunked counting sort from
// there on.
enum class Grouping { kOneBlock, kPerExpert, kChunked };
inline Grouping grouping_for(long n_pairs) {
  if (n_pairs <= kRouteSmallMax) return Grouping::kOneBlock;
  return n_pairs < kChunkSortMin ? Grouping::kPerExpert : Grouping::kChunked;
}

Layout layout_for(const moe_shape& s) {
  Layout L;
  const long np = (long)s.T * s.k;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.max_tiles = max_tiles_for(np, s.E, kSkinnyBM);
  L.max_tiles_big = max_tiles_for(np, s.E, tiles_bm(s));
  L.ctrl = take(sizeof(Ctrl));
  L.ids = take(np * 4);
  L.wts = take(np * 4);
  L.counts = take((size_t)s.E * 4);
  L.offsets = take((size_t)(s.E + 1) * 4);
  L.sorted = take(np * 4);
  L.inv = take(np * 4);
  L.tiles = take((size_t)(L.max_tiles + 1) * sizeof(Tile));
  L.tiles_big = take((size_t)(L.max_tiles_big + 1) * sizeof(Tile));
  const size_t n_chunks = (np + kSortChunk - 1) / kSortChunk;
  L.chunk_counts = take(n_chunks * s.E * 4);
  L.chunk_base = take(n_chunks * s.E * 4);
  L.rank = take(np * 4);
  const bool fp8 = s.wdtype == MOE_FP8_E4M3;
  L.xpart = take(fp8 ? kXParts * 4 : 0);
  L.xq = take(fp8 ? (size_t)s.T * s.H : 0);
  L.hq = take(fp8 ? (size_t)np * s.I : 0);
  L.h = take((size_t)np * s.I * act_bytes(s.wdtype));
  L.y = take((size_t)np * s.H * 4);
  L.max_rtiles = ((long)s.T + kRouterBM - 1) / kRouterBM;
  L.logits = take((size_t)s.T * s.E * 4);
  L.rtiles = take((size_t)(L.max_rtiles + 1) * sizeof(Tile));
  // last, so that adding it moved no other region (the GEMMs' speed
  // depends on where x, h and y sit)
  L.tiles_spread = take((size_t)(L.max_tiles_big + 1) * sizeof(Tile));
  L.total = o;
  return L;
}

// Workspace of moe_align_sort: control words, a tile list of <= kSkinnyBM
// positions (the one-block and chunked kernels form one) and the chunked
// sort's scratch.
struct AlignLayout {
  size_t ctrl, tiles, chunk_counts, chunk_base, rank, inv, total;
};

AlignLayout align_layout_for(int T, int k, int E) {
  AlignLayout L;
  const long np = (long)T * k;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.ctrl = take(sizeof(Ctrl));
  L.tiles = take((size_t)(max_tiles_for(np, E, kSkinnyBM) + 1) * sizeof(Tile));
  const size_t n_chunks = (np + kSortChunk - 1) / kSortChunk;
  L.chunk_counts = take(n_chunks * E * 4);
  L.chunk_base = take(n_chunks * E * 4);
  L.rank = take(np * 4);
  L.inv = take(np >= kChunkSortMin ? np * 4 : 0);
  L.total = o;
  return L;
}

template <typename T>
inline T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off);
}

int check_common(int T, int E, int k) {
  if (T < 0 || E < 1 || E > 1024 || k < 1 || k > 16 || k > E) return MOE_ERR_INVALID_ARG;
  if ((long)T * k >= (1L << 31)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int check_ws(const moe_shape* s, void* ws, size_t ws_bytes) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u)) return MOE_ERR_WORKSPACE;
  if (ws_bytes < moe_workspace_bytes(s)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                         \
  do {                                        \
    hipError_t _e = (expr);                   \
    if (_e != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

// Enqueue: per-tensor e4m3 quantisation of a bf16 tensor (amax, then codes).
int enqueue_quant(const uint16_t* src, long n, uint32_t* amax_bits, uint8_t* dst, hipStream_t st) {
  MOE_TRY(launch_amax_bf16(src, n, amax_bits, st));
  MOE_TRY(launch_quant_e4m3(src, n, amax_bits, dst, st));
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  int rc = check_common(s->T, s->E, s->k);
  if (rc) return rc;
  if (s->wdtype < MOE_F32 || s->wdtype > MOE_FP8_E4M3) return MOE_ERR_INVALID_ARG;
  if (s->renormalize != 0 && s->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (s->H <= 0 || s->I <= 0) return MOE_ERR_INVALID_ARG;
  if (s->H % 128 || s->I % 128) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t moe_workspace_bytes(const moe_shape* s) {
  if (moe_check_shape(s) != MOE_OK) return 0;
  return layout_for(*s).total;
}

int moe_workspace_routing(const moe_shape* s, moe_routing_offsets* out) {
  int rc = moe_check_shape(s);
  if (rc) return rc;
  if (!out) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_for(*s);
  out->topk_ids = L.ids;
  out->topk_weights = L.wts;
  out->expert_counts = L.counts;
  out->expert_offsets = L.offsets;
  out->sorted_ids = L.sorted;
  out->inv_perm = L.inv;
  return MOE_OK;
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape (H and I must be multiples of 128)";
    case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "HIP launch failure";
    case MOE_ERR_TOO_LARGE:
      return "shape needs more scratch than moe_fused_forward_noalloc's static buffer";
    default: return "unknown status";
  }
}

int moe_topk_gating(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renormalize,
                    int32_t* topk_ids, float* topk_weights, void* stream) {
  int rc = check_common(T, E, k);
  if (rc) return rc;
  if (renormalize != 0 && renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weights) return MOE_ERR_INVALID_ARG;
  if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_weights))
    return MOE_ERR_INVALID_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return hip_status(
      launch_topk_gating(logits, T, E, k, renormalize, topk_ids, topk_weights, nullptr, 0, st));
}

size_t moe_align_sort_workspace_bytes(int32_t T, int32_t k, int32_t E) {
  if (check_common(T, E, k) != MOE_OK) return 0;
  return align_layout_for(T, k, E).total;
}

int moe_align_sort(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                   int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_ids,
                   int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_common(T, E, k);
  if (rc) return rc;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !expert_counts || !expert_offsets || !sorted_ids) return MOE_ERR_INVALID_ARG;
  if (!aligned16(topk_ids) || !aligned16(expert_counts) || !aligned16(expert_offsets) ||
      !aligned16(sorted_ids) || (inv_perm && !aligned16(inv_perm)))
    return MOE_ERR_INVALID_ARG;
  const AlignLayout L = align_layout_for(T, k, E);
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u) || ws_bytes < L.total)
    return MOE_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const long n = (long)T * k;
  Ctrl* ctrl = at<Ctrl>(ws, L.ctrl);
  Tile* tiles = at<Tile>(ws, L.tiles);
  switch (grouping_for(n)) {
    case Grouping::kOneBlock:
      // ids are read, not written: the kernel's gating step is skipped
      return hip_status(launch_route_small(nullptr, T, E, k, 1, const_cast<int32_t*>(topk_ids),
                                           nullptr, expert_counts, expert_offsets, sorted_ids,
                                           inv_perm, kSkinnyBM, false, tiles, ctrl, nullptr, 0,
                                           nullptr, nullptr, nullptr, st));
    case Grouping::kPerExpert:
      return hip_status(launch_align_sort(topk_ids, T, k, E, expert_counts, expert_offsets,
                                          sorted_ids, inv_perm, st));
    case Grouping::kChunked: {
      // the chunked scatter always writes an inverse permutation; without the
      // caller's it goes to the workspace
      int32_t* inv = inv_perm ? inv_perm : at<int32_t>(ws, L.inv);
      return hip_status(launch_chunk_sort(topk_ids, (int)n, E, expert_counts, expert_offsets,
                                          sorted_ids, inv, kSkinnyBM, tiles, &ctrl->num_tiles,
                                          at<int32_t>(ws, L.chunk_counts),
                                          at<int32_t>(ws, L.chunk_base), at<int32_t>(ws, L.rank),
                                          st));
    }
  }
  return MOE_ERR_INVALID_ARG;
}

int moe_grouped_gemm_w13_swiglu(const moe_shape* s, const void* x, const void* w13,
                                const float* w13_scale, const int32_t* sorted_ids,
                                const int32_t* expert_offsets, void* h, float* act_scales,
                                void* ws, size_t ws_bytes, void* stream) {
  int rc = moe_check_shape(s);
  if (rc) return rc;
  if (s->T == 0) return MOE_OK;
  const bool fp8 = s->wdtype == MOE_FP8_E4M3;
  if (!x || !w13 || !sorted_ids || !expert_offsets || !h) return MOE_ERR_INVALID_ARG;
  if (fp8 && (!w13_scale || !act_scales)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w13) || !aligned16(sorted_ids) || !aligned16(expert_offsets) ||
      !aligned16(h) || (fp8 && (!aligned16(w13_scale) || !aligned16(act_scales))))
    return MOE_ERR_INVALID_ARG;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const Layout L = layout_for(*s);
  Ctrl* ctrl = at<Ctrl>(ws, L.ctrl);
  Tile* tiles = at<Tile>(ws, L.tiles);
  Tile* tiles_big = at<Tile>(ws, L.tiles_big);
  const bool big = use_tiles(*s);
  MOE_TRY(launch_zero_words(reinterpret_cast<uint32_t*>(ctrl), sizeof(Ctrl) / 4, st));
  if (big)
    MOE_TRY(launch_build_tiles(expert_offsets, s->E, tiles_bm(*s), tiles_big,
                               &ctrl->num_tiles_big, st));
  else
    MOE_TRY(launch_build_tiles(expert_offsets, s->E, kSkinnyBM, tiles, &ctrl->num_tiles, st));
  const void* b = x;
  if (fp8) {
    uint8_t* xq = at<uint8_t>(ws, L.xq);
    if ((rc = enqueue_quant(reinterpret_cast<const uint16_t*>(x), (long)s->T * s->H,
                            &ctrl->amax_x_bits, xq, st)))
      return rc;
    b = xq;
  }
  if (big)
    MOE_TRY(launch_w13_tiles(s->wdtype, tiles_bm(*s), b, w13, w13_scale, sorted_ids, tiles_big,
                             &ctrl->num_tiles_big, (int)L.max_tiles_big, s->H, s->I, s->k,
                             &ctrl->amax_x_bits, h, &ctrl->amax_h_bits, nullptr, nullptr, st));
  else
    MOE_TRY(launch_w13_swiglu(s->wdtype, b, w13, w13_scale, sorted_ids, tiles, ctrl,
                              (int)L.max_tiles, s->H, s->I, s->k, &ctrl->amax_x_bits, h,
                              &ctrl->amax_h_bits, nullptr, nullptr, st));
  if (fp8) MOE_TRY(launch_write_scales(ctrl, act_scales, st));
  return MOE_OK;
}

int moe_grouped_gemm_w2(const moe_shape* s, const void* h, const void* w2, const float* w2_scale,
                        const int32_t* expert_offsets, const float* act_scales, float* y,
                        void* ws, size_t ws_bytes, void* stream) {
  int rc = moe_check_shape(s);
  if (rc) return rc;
  if (s->T == 0) return MOE_OK;
  const bool fp8 = s->wdtype == MOE_FP8_E4M3;
  if (!h || !w2 || !expert_offsets || !y) return MOE_ERR_INVALID_ARG;
  if (fp8 && (!w2_scale || !act_scales)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w2) || !aligned16(expert_offsets) || !aligned16(y) ||
      (fp8 && (!aligned16(w2_scale) || !aligned16(act_scales))))
    return MOE_ERR_INVALID_ARG;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const Layout L = layout_for(*s);
  Ctrl* ctrl = at<Ctrl>(ws, L.ctrl);
  Tile* tiles = at<Tile>(ws, L.tiles);
  Tile* tiles_big = at<Tile>(ws, L.tiles_big);
  const bool big = use_tiles(*s);
  if (big)
    MOE_TRY(launch_build_tiles(expert_offsets, s->E, tiles_bm(*s), tiles_big,
                               &ctrl->num_tiles_big, st));
  else
    MOE_TRY(launch_build_tiles(expert_offsets, s->E, kSkinnyBM, tiles, &ctrl->num_tiles, st));
  const void* b = h;
  // act_scales[3] holds amax(h) as an fp32 value; its bit pattern is what the
  // kernels read.
  const uint32_t* amax_h = reinterpret_cast<const uint32_t*>(fp8 ? act_scales + 3 : nullptr);
  if (fp8) {
    uint8_t* hq = at<uint8_t>(ws, L.hq);
    MOE_TRY(launch_quant_e4m3(reinterpret_cast<const uint16_t*>(h), (long)s->T * s->k * s->I,
                              amax_h, hq, st));
    b = hq;
  }
  if (big)
    MOE_TRY(launch_w2_tiles(s->wdtype, tiles_bm(*s), b, w2, w2_scale, tiles_big,
                            &ctrl->num_tiles_big, (int)L.max_tiles_big, s->H, s->I, amax_h, y,
                            false, nullptr, nullptr, st));
  else
    MOE_TRY(launch_w2(s->wdtype, b, w2, w2_scale, tiles, ctrl, (int)L.max_tiles, s->H, s->I,
                      amax_h, y, nullptr, nullptr, st));
  return MOE_OK;
}

int moe_act_quant_e4m3(const void* a, int64_t n, uint8_t* codes, float* scales, void* stream) {
  if (n == 0) return MOE_OK;
  if (n < 0 || n % 8 || !a || !codes || !scales) return MOE_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(codes) || !aligned16(scales)) return MOE_ERR_INVALID_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // scales[1] takes the amax bits (integer atomics on fp32 patterns), then
  // the value they encode; scales[0] the scale
  uint32_t* amax_bits = reinterpret_cast<uint32_t*>(scales + 1);
  MOE_TRY(launch_zero_words(amax_bits, 1, st));
  MOE_TRY(launch_amax_bf16(reinterpret_cast<const uint16_t*>(a), (long)n, amax_bits, st));
  MOE_TRY(launch_quant_e4m3(reinterpret_cast<const uint16_t*>(a), (long)n, amax_bits, codes, st));
  MOE_TRY(launch_finish_scale(scales, st));
  return MOE_OK;
}

int moe_inv_rope_fp8_quant(const void* x, const int32_t* positions, const float* cos_sin,
                           int32_t T, int32_t n_heads, int32_t head_dim, int32_t rot_dim,
                           int32_t max_pos, int32_t interleaved, uint8_t* codes, float* scales,
                           void* stream) {
  if (T < 0 || n_heads < 1 || max_pos < 1 || (interleaved != 0 && interleaved != 1))
    return MOE_ERR_INVALID_ARG;
  if ((long)T * n_heads >= (1L << 31)) return MOE_ERR_INVALID_ARG;
  if (head_dim % 16 || head_dim < 16 || head_dim > 512 || rot_dim % 16 || rot_dim < 16 ||
      rot_dim > head_dim)
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !positions || !cos_sin || !codes || !scales) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(positions) || !aligned16(cos_sin) || !aligned16(codes) ||
      !aligned16(scales))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_inv_rope_fp8(reinterpret_cast<const uint16_t*>(x), positions, cos_sin,
                                        T, n_heads, head_dim, rot_dim, max_pos, interleaved != 0,
                                        codes, scales, reinterpret_cast<hipStream_t>(stream)));
}

int moe_combine(const moe_shape* s, const float* y, const int32_t* inv_perm,
                const float* topk_weights, void* out, void* stream) {
  int rc = moe_check_shape(s);
  if (rc) return rc;
  if (s->T == 0) return MOE_OK;
  if (!y || !inv_perm || !topk_weights || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y) || !aligned16(inv_perm) || !aligned16(topk_weights) || !aligned16(out))
    return MOE_ERR_INVALID_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return hip_status(
      launch_combine(s->wdtype, y, false, inv_perm, topk_weights, s->T, s->H, s->k, out, st));
}

}  // extern "C"

namespace {

int router_impl(const moe_shape* s, const void* x, const void* wg, float* logits, void* ws,
                hipStream_t st) {
  const Layout L = layout_for(*s);
  Ctrl* ctrl = at<Ctrl>(ws, L.ctrl);
  return hip_status(launch_router_logits(s->wdtype, x, wg, s->T, s->H, s->E, logits,
                                         at<Tile>(ws, L.rtiles), &ctrl->num_tiles_router,
                                         (int)L.max_rtiles, st));
}

int check_router_args(const moe_shape* s, const void* x, const void* wg, const float* logits) {
  if (!x || !wg) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(wg) || (logits && !aligned16(logits)))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_router_logits(const moe_shape* s, const void* x, const void* wg, float* logits, void* ws,
                      size_t ws_bytes, void* stream) {
  int rc = moe_check_shape(s);
  if (rc) return rc;
  if (s->T == 0) return MOE_OK;
  if (!logits) return MOE_ERR_INVALID_ARG;
  if ((rc = check_router_args(s, x, wg, logits))) return rc;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  return router_impl(s, x, wg, logits, ws, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Argument checks of the fused entry points (shape already valid, T > 0).
int check_fused_args(const moe_shape* s, const void* x, const float* logits, const void* w13,
                     const float* w13_scale, const void* w2, const float* w2_scale,
                     const void* out, const int32_t* topk_ids, const float* topk_weights,
                     void* ws, size_t ws_bytes) {
  const bool fp8 = s->wdtype == MOE_FP8_E4M3;
  if (!x || !logits || !w13 || !w2 || !out) return MOE_ERR_INVALID_ARG;
  if (fp8 && (!w13_scale || !w2_scale)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(logits) || !aligned16(w13) || !aligned16(w2) ||
      !aligned16(out) || (topk_ids && !aligned16(topk_ids)) ||
      (topk_weights && !aligned16(topk_weights)) ||
      (fp8 && (!aligned16(w13_scale) || !aligned16(w2_scale))))
    return MOE_ERR_INVALID_ARG;
  return check_ws(s, ws, ws_bytes);
}

// Router fused into the front kernel: bf16 router weights (BF16 and FP8
// layers) small enough for one block to stream, a batch the one-block front
// takes, and logits that fit its LDS.
inline bool router_in_front(const moe_shape& s) {
  return s.wdtype != MOE_F32 && grouping_for((long)s.T * s.k) == Grouping::kOneBlock &&
         (long)s.T * s.E <= kFusedRouterMaxTE && (long)s.E * s.H <= kFusedRouterMaxEH;
}

// The layer.  With wg (only when router_in_front), the front kernel computes
// the logits from x and wg itself and copies them to logits_out if given;
// `logits` is then unused.
int fused_impl(const moe_shape* s, const void* x, const float* logits, const void* w13,
               const float* w13_scale, const void* w2, const float* w2_scale, void* out,
               int32_t* topk_ids, float* topk_weights, void* ws, size_t ws_bytes, void* stream,
               void** events, const void* wg = nullptr, float* logits_out = nullptr) {
  int rc = moe_check_shape(s);
  if (rc) return rc;
  if (s->T == 0) return MOE_OK;
  const bool fp8 = s->wdtype == MOE_FP8_E4M3;
  if ((rc = check_fused_args(s, x, logits, w13, w13_scale, w2, w2_scale, out, topk_ids,
                             topk_weights, ws, ws_bytes)))
    return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // boundaries 0-3 and 8 are marker events; 4/5 and 6/7 are the start / end
  // of the gate/up and down GEMM dispatches themselves
  auto ev = [&](int i) -> hipEvent_t {
    return events ? reinterpret_cast<hipEvent_t>(events[i]) : nullptr;
  };
  auto mark = [&](int i) -> hipError_t {
    return ev(i) ? hipEventRecord(ev(i), st) : hipSuccess;
  };
  const Layout L = layout_for(*s);
  const int T = s->T, H = s->H, E = s->E, k = s->k, I = s->I;
  Ctrl* ctrl = at<Ctrl>(ws, L.ctrl);
  int32_t* ids = topk_ids ? topk_ids : at<int32_t>(ws, L.ids);
  float* wts = topk_weights ? topk_weights : at<float>(ws, L.wts);
  int32_t* counts = at<int32_t>(ws, L.counts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* sorted = at<int32_t>(ws, L.sorted);
  int32_t* inv = at<int32_t>(ws, L.inv);
  Tile* tiles = at<Tile>(ws, L.tiles);
  Tile* tiles_big = at<Tile>(ws, L.tiles_big);
  const bool big = use_tiles(*s);
  void* h = at<void>(ws, L.h);
  float* y = at<float>(ws, L.y);

  const Grouping grouping = grouping_for((long)T * k);
  uint8_t* xq = fp8 ? at<uint8_t>(ws, L.xq) : nullptr;
  const void* bx = fp8 ? static_cast<const void*>(xq) : x;

  const int bm = big ? tiles_bm(*s) : kSkinnyBM;
  Tile* tl = big ? tiles_big : tiles;
  // The down projection's tiles in the spread order (full 128-position tiles
  // evenly among the partial ones), written by the chunked grouping beside
  // the expert-ordered list, while experts average fewer than 256 pairs (so
  // that many of their tiles are partial).  Measured on the prefill layer
  // (128 pairs per expert, Zipf): down projection 1.11-1.12 -> 1.04-1.05 ms,
  // layer 3.19 -> 3.14 ms per step; at 512 pairs per expert (16k tokens, 87%
  // of the tiles full) the down projection was unchanged and the placement
  // cost the grouping 9 us.  The gate/up projection keeps the expert order,
  // which was 6% faster for it (an expert's tiles run side by side and share
  // its weight rows in L2).
  const bool spread = big && bm == 128 && grouping == Grouping::kChunked &&
                      (long)T * k < 256L * E;
  Tile* tiles_w2 = spread ? at<Tile>(ws, L.tiles_spread) : tiles_big;
  MOE_TRY(mark(0));
  if (grouping == Grouping::kOneBlock) {
    // the front kernel's second block quantises a small x; a large one goes
    // to the grid-wide passes after it (the kernel leaves amax(x) at 0)
    const bool front_quant = fp8 && (long)T * H <= kFrontQuantMax;
    MOE_TRY(launch_route_small(wg ? nullptr : logits, T, E, k, s->renormalize, ids, wts, counts,
                               offsets, sorted, inv, bm, big, tl, ctrl,
                               reinterpret_cast<const uint16_t*>(x), H,
                               front_quant ? xq : nullptr,
                               reinterpret_cast<const uint16_t*>(wg), logits_out, st));
    for (int i = 1; i <= 3; i++) MOE_TRY(mark(i));
    if (fp8 && !front_quant &&
        (rc = enqueue_quant(reinterpret_cast<const uint16_t*>(x), (long)T * H, &ctrl->amax_x_bits,
                            xq, st)))
      return rc;
  } else {
    // FP8: the quantisation of x rides along in extra blocks of the gating
    // launch (partial maxima of |x|) and of the grouping launch (amax(x) and
    // the codes), beside their latency-bound work
    const XWork xw{reinterpret_cast<const uint16_t*>(x), (long)T * H / 8, at<float>(ws, L.xpart),
                   ctrl, xq};
    const XWork* xwp = fp8 ? &xw : nullptr;
    // zeroes the control block
    MOE_TRY(launch_topk_gating(logits, T, E, k, s->renormalize, ids, wts,
                               reinterpret_cast<uint32_t*>(ctrl), sizeof(Ctrl) / 4, st, xwp));
    MOE_TRY(mark(1));
    int32_t* nt = big ? &ctrl->num_tiles_big : &ctrl->num_tiles;
    if (grouping == Grouping::kChunked) {
      MOE_TRY(launch_chunk_sort(ids, T * k, E, counts, offsets, sorted, inv, bm, tl, nt,
                                at<int32_t>(ws, L.chunk_counts), at<int32_t>(ws, L.chunk_base),
                                at<int32_t>(ws, L.rank), st, xwp, spread ? tiles_w2 : nullptr));
      MOE_TRY(mark(2));
    } else {
      MOE_TRY(launch_align_sort(ids, T, k, E, counts, offsets, sorted, inv, st, xwp));
      MOE_TRY(mark(2));
      MOE_TRY(launch_build_tiles(offsets, E, bm, tl, nt, st));
    }
    MOE_TRY(mark(3));
  }
  if (big)
    MOE_TRY(launch_w13_tiles(s->wdtype, tiles_bm(*s), bx, w13, w13_scale, sorted, tiles_big,
                             &ctrl->num_tiles_big, (int)L.max_tiles_big, H, I, k,
                             &ctrl->amax_x_bits, h, &ctrl->amax_h_bits, ev(4), ev(5), st));
  else
    MOE_TRY(launch_w13_swiglu(s->wdtype, bx, w13, w13_scale, sorted, tiles, ctrl,
                              (int)L.max_tiles, H, I, k, &ctrl->amax_x_bits, h,
                              &ctrl->amax_h_bits, ev(4), ev(5), st));
  const void* bh = h;
  if (fp8) {
    uint8_t* hq = at<uint8_t>(ws, L.hq);
    MOE_TRY(launch_quant_e4m3(reinterpret_cast<const uint16_t*>(h), (long)T * k * I,
                              &ctrl->amax_h_bits, hq, st));
    bh = hq;
  }
  // FP8 layers with many tokens per expert keep y in bf16 between the down
  // projection and the aggregation (half the bytes of that round trip); the
  // step entry points return fp32 y
  const bool y_bf16 = fp8 && big;
  if (big)
    MOE_TRY(launch_w2_tiles(s->wdtype, tiles_bm(*s), bh, w2, w2_scale, tiles_w2,
                            &ctrl->num_tiles_big, (int)L.max_tiles_big, H, I, &ctrl->amax_h_bits,
                            y, y_bf16, ev(6), ev(7), st));
  else
    MOE_TRY(launch_w2(s->wdtype, bh, w2, w2_scale, tiles, ctrl, (int)L.max_tiles, H, I,
                      &ctrl->amax_h_bits, y, ev(6), ev(7), st));
  MOE_TRY(launch_combine(s->wdtype, y, y_bf16, inv, wts, T, H, k, out, st));
  MOE_TRY(mark(8));
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_fused_forward_router(const moe_shape* s, const void* x, const void* wg, const void* w13,
                             const float* w13_scale, const void* w2, const float* w2_scale,
                             void* out, float* logits, int32_t* topk_ids, float* topk_weights,
                             void* ws, size_t ws_bytes, void* stream) {
  int rc = moe_check_shape(s);
  if (rc) return rc;
  if (s->T == 0) return MOE_OK;
  if ((rc = check_router_args(s, x, wg, logits))) return rc;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  float* lg = logits ? logits : at<float>(ws, layout_for(*s).logits);
  // every argument of the layer is checked before anything is enqueued
  if ((rc = check_fused_args(s, x, lg, w13, w13_scale, w2, w2_scale, out, topk_ids,
                             topk_weights, ws, ws_bytes)))
    return rc;
  // few-token batches: one front kernel computes the logits, gates and
  // groups (no router launch, the logits stay on chip)
  if (router_in_front(*s))
    return fused_impl(s, x, lg, w13, w13_scale, w2, w2_scale, out, topk_ids, topk_weights, ws,
                      ws_bytes, stream, nullptr, wg, logits);
  if ((rc = router_impl(s, x, wg, lg, ws, reinterpret_cast<hipStream_t>(stream)))) return rc;
  return fused_impl(s, x, lg, w13, w13_scale, w2, w2_scale, out, topk_ids, topk_weights, ws,
                    ws_bytes, stream, nullptr);
}

int moe_fused_forward(const moe_shape* s, const void* x, const float* logits, const void* w13,
                      const float* w13_scale, const void* w2, const float* w2_scale, void* out,
                      int32_t* topk_ids, float* topk_weights, void* ws, size_t ws_bytes,
                      void* stream) {
  return fused_impl(s, x, logits, w13, w13_scale, w2, w2_scale, out, topk_ids, topk_weights, ws,
                    ws_bytes, stream, nullptr);
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup fails.
static void* noalloc_scratch() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  static bool done[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!done[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptr[dev] = p;
    done[dev] = true;
  }
  return ptr[dev];
}

int moe_fused_forward_noalloc(const moe_shape* s, const void* x, const float* logits,
                              const void* w13, const float* w13_scale, const void* w2,
                              const float* w2_scale, void* out, int32_t* topk_ids,
                              float* topk_weights, void* stream) {
  int rc = moe_check_shape(s);
  if (rc) return rc;
  if (s->T == 0) return MOE_OK;
  if (moe_workspace_bytes(s) > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_TOO_LARGE;
  void* ws = noalloc_scratch();
  if (!ws) return MOE_ERR_HIP;
  // the kernels clear what must start at zero (the control words) themselves
  return fused_impl(s, x, logits, w13, w13_scale, w2, w2_scale, out, topk_ids, topk_weights, ws,
                    (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int moe_fused_forward_events(const moe_shape* s, const void* x, const float* logits,
                             const void* w13, const float* w13_scale, const void* w2,
                             const float* w2_scale, void* out, int32_t* topk_ids,
                             float* topk_weights, void* ws, size_t ws_bytes, void* stream,
                             void** events, int32_t n_events) {
  if (!events || n_events != MOE_NUM_STAGE_EVENTS) return MOE_ERR_INVALID_ARG;
  return fused_impl(s, x, logits, w13, w13_scale, w2, w2_scale, out, topk_ids, topk_weights, ws,
                    ws_bytes, stream, events);
}

}  // extern "C"
