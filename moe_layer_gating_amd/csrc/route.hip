// route.hip -- token routing and grouping kernels of the fused MoE layer.
//
// Routing (top-k softmax gating) and the regrouping of (token, slot) pairs into
// expert-contiguous order are the "token routing" and "data shuffling" stages
// of the fused MoE operation (readmex.ai, "AWS details fused MoE kernel
// optimizations on SageMaker, up to 10% throughput gain", summary).  Both stay
// on the device so that no host round-trip sits between them and the expert
// GEMMs (explore.n1n.ai, "Mixture-of-Experts Kernel Engineering on Amazon
// SageMaker AI", section "2. Triton Backend Routing for FP8 Quantization").
// Per-expert batch sizes are data dependent (same page, "The Core
// Bottlenecks of MoE Inference on H200 GPUs"): they are produced here as
// counts / offsets / a tile list that the GEMMs read on the device, so no
// kernel is specialised on them.
#include "moe_common.h"

namespace moe {

// ---------------------------------------------------------------- gating
// One wave per token.  Lane l holds logits e = l, l+64, ... (up to 16 each).
// k rounds of a wave-wide arg-max over the experts not yet taken; the order
// is (logit descending, expert index ascending).  Float comparison makes
// -0 == +0.  After round j, lane j keeps the winner, so lanes 0..k-1 end up
// holding slot j's (value, expert).
constexpr int kMaxPerLane = 16;  // E <= 1024

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// LDS words of the per-wave scratch of gate_token's rank selection: the
// token's selection keys (two 64-bit keys per lane), then k slot values and
// k slot experts.
constexpr int kRankMaxE = 2 * kWave;
constexpr int kGateScratch = 2 * kRankMaxE + 2 * 16;

// Selection key of expert e with logit v: larger key = earlier in the order
// (logit descending, expert index ascending).  The high word maps the float
// to an unsigned integer of the same order (-0 first made +0, so the two
// zeros tie as they compare equal), the low word is ~e.
__device__ __forceinline__ uint64_t gate_key(float v, int e) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)~e;
}

// Orders this wave's LDS accesses: every lane's earlier LDS writes are
// complete and visible to the other lanes before any later access.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Top-k of one token by one whole wave; lanes 0..k-1 write slot `lane` to
// ids_row / wts_row (and to lds_ids if given).  With `scratch` (kGateScratch
// words of LDS owned by this wave, 8-byte aligned) and E <= kRankMaxE the
// selection is by ranks: the selection keys of the row (gate_key) go to LDS
// and every lane counts, for each of its (one, or two when E > 64) logits,
// the keys larger than its own, reading them back two at a time (broadcast
// reads); the logit of rank j < k is slot j.  That is one pass of
// independent 64-bit comparisons instead of k dependent wave-wide arg-max
// rounds, and selects the same experts.
__device__ __forceinline__ void gate_token(const float* __restrict__ row, int E, int k, int renorm,
                                           int32_t* __restrict__ ids_row,
                                           float* __restrict__ wts_row, int* lds_ids,
                                           float* scratch = nullptr) {
  const int lane = lane_id();
  float v[kMaxPerLane];
  const int per_lane = (E + kWave - 1) / kWave;
  // A NaN logit breaks the contract; it is read as -inf so that a violation
  // still selects experts inside [0, E) (every candidate, -inf included, is
  // ordered by (value, index)), rather than an index the grouping would use
  // out of bounds.
#pragma unroll
  for (int i = 0; i < kMaxPerLane; i++) {
    int e = lane + i * kWave;
    const float lv = (i < per_lane && e < E) ? row[e] : -INFINITY;
    v[i] = (lv == lv) ? lv : -INFINITY;
  }
  uint32_t taken = 0;  // bit i: slot i of this lane already selected (or absent)
#pragma unroll
  for (int i = 0; i < kMaxPerLane; i++)
    if (!(i < per_lane && lane + i * kWave < E)) taken |= 1u << i;

  float my_v = -INFINITY, top_v = 0.f;
  int my_e = 0;
  if (scratch && E <= kRankMaxE) {
    uint64_t* skey = reinterpret_cast<uint64_t*>(scratch);
    float* sv = scratch + 2 * kRankMaxE;
    int* se = reinterpret_cast<int*>(scratch + 2 * kRankMaxE + 16);
    wave_lds_sync();  // a previous token's reads of this scratch are done
    // v[i] is -inf beyond E: such an entry has an index >= E, so its key is
    // below every real expert's, and its own rank is at least E >= k
    const uint64_t k0 = gate_key(v[0], lane), k1 = gate_key(v[1], lane + kWave);
    skey[lane] = k0;
    skey[lane + kWave] = k1;
    wave_lds_sync();
    int r0 = 0, r1 = 0;
    typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
    const u64x2* s2 = reinterpret_cast<const u64x2*>(skey);
    // eight 16-byte reads per round; rounds past E read the padding keys
    // (all kRankMaxE are written), which never exceed a real expert's key
    const int nq = (E + 1) / 2;
    if (E > kWave) {
      for (int q0 = 0; q0 < nq; q0 += 8) {
        u64x2 c[8];
#pragma unroll
        for (int u = 0; u < 8; u++) c[u] = s2[q0 + u];
#pragma unroll
        for (int u = 0; u < 8; u++) {
          r0 += (c[u][0] > k0) + (c[u][1] > k0);
          r1 += (c[u][0] > k1) + (c[u][1] > k1);
        }
      }
    } else {
      for (int q0 = 0; q0 < nq; q0 += 8) {
        u64x2 c[8];
#pragma unroll
        for (int u = 0; u < 8; u++) c[u] = s2[q0 + u];
#pragma unroll
        for (int u = 0; u < 8; u++) r0 += (c[u][0] > k0) + (c[u][1] > k0);
      }
      r1 = kRankMaxE;  // the second slot is padding
    }
    if (lane < E && r0 < k) {
      sv[r0] = v[0];
      se[r0] = lane;
    }
    if (lane + kWave < E && r1 < k) {
      sv[r1] = v[1];
      se[r1] = lane + kWave;
    }
    wave_lds_sync();
    top_v = sv[0];
    if (lane < k) {
      my_v = sv[lane];
      my_e = se[lane];
    }
  } else {
  for (int j = 0; j < k; j++) {
    // best untaken candidate of this lane
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; i++) {
      int e = lane + i * kWave;
      if (!(taken & (1u << i)) && better(v[i], e, bv, be)) {
        bv = v[i];
        be = e;
      }
    }
    // butterfly arg-max: every lane ends with the wave winner
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      float ov = __shfl_xor(bv, o);
      int oe = __shfl_xor(be, o);
      if (better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if (be < E && (be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
    if (j == 0) top_v = bv;
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
  }
  }
  // weights: exp(l - l_top) over the selected slots, divided by their sum
  // (renorm) or by the sum over every expert (top_v is the row maximum).
  float ex = (lane < k) ? expf(my_v - top_v) : 0.f;
  float denom;
  if (renorm) {
    denom = wave_sum(ex);
  } else {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; i++)
      if (i < per_lane && lane + i * kWave < E) s += expf(v[i] - top_v);
    denom = wave_sum(s);
  }
  if (lane < k) {
    ids_row[lane] = my_e;
    wts_row[lane] = ex / denom;
    if (lds_ids) lds_ids[lane] = my_e;
  }
}

// ------------------------------------------------- x work of extra blocks
// Block b of nb (any block size up to 1024): max |x| over its grid-stride
// slice into xw.part[b], four 16-byte loads in flight per thread.
__device__ __forceinline__ void x_amax_part(const XWork& xw, int b, int nb) {
  __shared__ float red[16];
  const i32x4* s4 = reinterpret_cast<const i32x4*>(xw.x);
  const long stride = (long)nb * blockDim.x;
  float m = 0.f;
  for (long i0 = (long)b * blockDim.x + threadIdx.x; i0 < xw.n8; i0 += 4 * stride) {
    i32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const long i = i0 + u * stride;
      v[u] = i < xw.n8 ? s4[i] : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 4; u++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const uint32_t w = (uint32_t)v[u][q];
        m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(w & 0xffffu))));
        m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(w >> 16))));
      }
  }
  m = wave_max(m);
  if (lane_id() == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = red[0];
    for (int i = 1; i < (int)(blockDim.x / kWave); i++) a = fmaxf(a, red[i]);
    xw.part[b] = a;
  }
}

// Block b of nb: amax(x) from the kXParts partials (block 0 stores it in
// the control block), then the e4m3 codes of its grid-stride slice (the
// rule of quant_e4m3_kernel: codes of fl32(x * fl32(448 / amax))).
__device__ __forceinline__ void x_quant_part(const XWork& xw, int b, int nb) {
  __shared__ float red[16];
  float a = 0.f;
  for (int i = threadIdx.x; i < kXParts; i += blockDim.x) a = fmaxf(a, xw.part[i]);
  a = wave_max(a);
  if (lane_id() == 0) red[threadIdx.x / kWave] = a;
  __syncthreads();
  a = red[0];
  for (int i = 1; i < (int)(blockDim.x / kWave); i++) a = fmaxf(a, red[i]);
  if (b == 0 && threadIdx.x == 0) xw.ctrl->amax_x_bits = __float_as_uint(a);
  const float r = a > 0.f ? 448.0f / a : 1.0f;
  const i32x4* s4 = reinterpret_cast<const i32x4*>(xw.x);
  uint2* d2 = reinterpret_cast<uint2*>(xw.xq);
  const long stride = (long)nb * blockDim.x;
  for (long i0 = (long)b * blockDim.x + threadIdx.x; i0 < xw.n8; i0 += 4 * stride) {
    i32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const long i = i0 + u * stride;
      v[u] = i < xw.n8 ? s4[i] : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const long i = i0 + u * stride;
      if (i < xw.n8) d2[i] = bf16x8_to_e4m3x8(v[u], r);
    }
  }
}

__global__ __launch_bounds__(256) void topk_gating_kernel(const float* __restrict__ logits, int T,
                                                          int E, int k, int renorm,
                                                          int32_t* __restrict__ ids,
                                                          float* __restrict__ wts,
                                                          uint32_t* zero_words, int n_zero,
                                                          int gate_blocks, XWork xw) {
  __shared__ __attribute__((aligned(16))) float gscr[4][kGateScratch];
  if ((int)blockIdx.x >= gate_blocks) {  // block-uniform
    x_amax_part(xw, blockIdx.x - gate_blocks, kXParts);
    return;
  }
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_zero; i += blockDim.x) zero_words[i] = 0u;
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  gate_token(logits + (size_t)t * E, E, k, renorm, ids + (size_t)t * k, wts + (size_t)t * k,
             nullptr, gscr[threadIdx.x / kWave]);
}

hipError_t launch_topk_gating(const float* logits, int T, int E, int k, int renorm, int32_t* ids,
                              float* w, uint32_t* zero_words, int n_zero, hipStream_t st,
                              const XWork* xw) {
  const int tokens_per_block = 4;
  int grid = (T + tokens_per_block - 1) / tokens_per_block;
  if (grid < 1) grid = 1;
  topk_gating_kernel<<<grid + (xw ? kXParts : 0), 256, 0, st>>>(
      logits, T, E, k, renorm, ids, w, zero_words, n_zero, grid, xw ? *xw : XWork{});
  return hipGetLastError();
}

// ------------------------------------------------------------ block scans
// Exclusive scan of one int per thread over a 256-thread block; returns the
// prefix and writes the block total to *total.  `tmp` holds 4 ints of LDS.
__device__ __forceinline__ int block_exclusive_scan_256(int v, int* tmp, int* total) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int n = __shfl_up(incl, o);
    if (lane >= o) incl += n;
  }
  if (lane == kWave - 1) tmp[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    int c = tmp[i];
    if (i < w) base += c;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// -------------------------------------------------------------- align sort
// grid = E blocks of 256 threads.  Every block builds the full expert
// histogram in LDS (integer atomics: the counts do not depend on order) and
// its exclusive scan, then block e gathers the pairs routed to expert e in
// ascending pair order with a ballot-based stable compaction.  No atomic
// decides a position, so the permutation is the same on every run.
__global__ __launch_bounds__(256) void align_sort_kernel(const int32_t* __restrict__ ids, int n,
                                                         int E, int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ sorted_ids,
                                                         int32_t* __restrict__ inv_perm,
                                                         XWork xw) {
  __shared__ int hist[1024];
  __shared__ int tmp[4];
  if ((int)blockIdx.x >= E) {  // block-uniform: the x encoding blocks
    x_quant_part(xw, blockIdx.x - E, kXQuantBlocks);
    return;
  }
  const int e = blockIdx.x;
  for (int i = threadIdx.x; i < E; i += 256) hist[i] = 0;
  __syncthreads();
  for (int f = threadIdx.x; f < n; f += 256) atomicAdd(&hist[ids[f]], 1);
  __syncthreads();
  // exclusive scan over E (<= 1024): thread i owns entries 4i .. 4i+3
  int local[4], s = 0;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    int idx = threadIdx.x * 4 + q;
    local[q] = (idx < E) ? hist[idx] : 0;
    s += local[q];
  }
  int total;
  int pre = block_exclusive_scan_256(s, tmp, &total);
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; q++) {
    int idx = threadIdx.x * 4 + q;
    if (idx < E) hist[idx] = pre;  // hist now holds the exclusive offsets
    pre += local[q];
  }
  __syncthreads();
  const int base = hist[e];
  const int cnt = (e + 1 < E ? hist[e + 1] : n) - base;
  if (threadIdx.x == 0) {
    counts[e] = cnt;
    offsets[e] = base;
    if (e == E - 1) offsets[E] = n;
  }
  if (cnt == 0) return;
  const int lane = lane_id(), w = threadIdx.x / kWave;
  int running = 0;
  for (int c0 = 0; c0 < n; c0 += 256) {
    int f = c0 + threadIdx.x;
    bool flag = (f < n) && ids[f] == e;
    uint64_t m = __ballot(flag);
    int rank = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) tmp[w] = __popcll(m);
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      int cw = tmp[i];
      if (i < w) before += cw;
      tot += cw;
    }
    if (flag) {
      int pos = base + running + before + rank;
      sorted_ids[pos] = f;
      if (inv_perm) inv_perm[f] = pos;
    }
    running += tot;
    __syncthreads();
    if (running == cnt) break;  // uniform across the block
  }
}

hipError_t launch_align_sort(const int32_t* ids, int T, int k, int E, int32_t* counts,
                             int32_t* offsets, int32_t* sorted_ids, int32_t* inv_perm,
                             hipStream_t st, const XWork* xw) {
  align_sort_kernel<<<E + (xw ? kXQuantBlocks : 0), 256, 0, st>>>(
      ids, T * k, E, counts, offsets, sorted_ids, inv_perm, xw ? *xw : XWork{});
  return hipGetLastError();
}

// -------------------------------------------------------------- tile list
// One block of 256 threads.  Expert e with c = offsets[e+1]-offsets[e] pairs
// contributes ceil(c / bm) tiles of at most bm consecutive sorted positions;
// tiles are listed expert by expert.  The tile count goes to *num_tiles.
__global__ __launch_bounds__(256) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                          int E,
                                                          int bm, Tile* __restrict__ tiles,
                                                          int32_t* num_tiles) {
  __shared__ int tmp[4];
  int local[4], s = 0;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    int e = threadIdx.x * 4 + q;
    int c = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    local[q] = (c + bm - 1) / bm;
    s += local[q];
  }
  int total;
  int pre = block_exclusive_scan_256(s, tmp, &total);
#pragma unroll
  for (int q = 0; q < 4; q++) {
    int e = threadIdx.x * 4 + q;
    if (e < E) {
      int p = offsets[e], end = offsets[e + 1];
      for (int i = 0; i < local[q]; i++) {
        Tile tl;
        tl.e = e;
        tl.p0 = p + i * bm;
        tl.mt = min(bm, end - tl.p0);
        tl.pad = 0;
        tiles[pre + i] = tl;
      }
    }
    pre += local[q];
  }
  if (threadIdx.x == 0) *num_tiles = total;
}

hipError_t launch_build_tiles(const int32_t* offsets, int E, int bm, Tile* tiles,
                              int32_t* num_tiles, hipStream_t st) {
  build_tiles_kernel<<<1, 256, 0, st>>>(offsets, E, bm, tiles, num_tiles);
  return hipGetLastError();
}

__global__ void zero_words_kernel(uint32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_zero_words(uint32_t* p, int n, hipStream_t st) {
  zero_words_kernel<<<(n + 255) / 256, 256, 0, st>>>(p, n);
  return hipGetLastError();
}

// ------------------------------------------------ router inside the front
// The router GEMM of a small batch, computed by the front kernel itself so
// that the gating reads the logits from LDS: no router launch in front and no
// logits round trip through HBM (token routing as the first stage of the one
// fused operation: readmex.ai, "AWS details fused MoE kernel optimizations on
// SageMaker, up to 10% throughput gain", summary; routing logic kept inside
// the fused kernels rather than in separate steps: explore.n1n.ai,
// "Mixture-of-Experts Kernel Engineering on Amazon SageMaker AI", section
// "2. Triton Backend Routing for FP8 Quantization").
//
// lgs[t * E + e] = x[t] . wg[e] for t < T, e < E (x [T,H], wg [E,H] bf16).
// bf16 MFMA (v_mfma_f32_16x16x32_bf16): experts on the row side, tokens on
// the column side, 16 x 16 output tiles; exact products, fp32 sums.  A work
// item is up to 4 expert tiles of one token tile (the token fragment loaded
// once for all 4) over a range of K.  With few items the 16 waves split K
// into `parts` ranges and the partial tiles are added through LDS in range
// order, one expert tile at a time; otherwise each wave takes whole items.
// Every lane loads 16 bytes (8 values) of K per step from one row of each
// operand, at the same K offsets on both sides.
__device__ __forceinline__ void router_logits_block(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ wg, int T, int H,
                                                    int E, float* lgs, float (*part)[256]) {
  constexpr int NW = 16, U = 2;
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int n_et = (E + 15) / 16, n_tt = (T + 15) / 16;
  const int n_eg = (n_et + 3) / 4, n_groups = n_eg * n_tt;
  const int n_steps = H / 32;
  int parts = NW / n_groups;
  parts = parts < 1 ? 1 : (parts > n_steps ? n_steps : parts);
  const i32x4 z4 = {0, 0, 0, 0};
  for (int base = 0; base < n_groups * parts; base += NW) {  // uniform over the block
    const int item = base + w;
    const bool live = item < n_groups * parts;
    const int grp = live ? item / parts : 0, p = live ? item - grp * parts : 0;
    const int eg = grp % n_eg, tt = grp / n_eg;
    const int t = tt * 16 + r;
    const bool vt = live && t < T;
    const char* brow = reinterpret_cast<const char*>(x + (size_t)(vt ? t : 0) * H) + g * 16;
    const char* arow[4];
    bool ve[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int e = (eg * 4 + q) * 16 + r;
      ve[q] = live && e < E;
      arow[q] = reinterpret_cast<const char*>(wg + (size_t)(ve[q] ? e : 0) * H) + g * 16;
    }
    f32x4 acc[4];
#pragma unroll
    for (int q = 0; q < 4; q++) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int s0 = live ? (int)((long)p * n_steps / parts) : 0;
    const int s1 = live ? (int)((long)(p + 1) * n_steps / parts) : 0;
    for (int s = s0; s < s1; s += U) {
      i32x4 a[U][4], b[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const bool in = s + u < s1;
        const size_t off = (size_t)(s + u) * 64;
        b[u] = (in && vt) ? *reinterpret_cast<const i32x4*>(brow + off) : z4;
#pragma unroll
        for (int q = 0; q < 4; q++)
          a[u][q] = (in && ve[q]) ? *reinterpret_cast<const i32x4*>(arow[q] + off) : z4;
      }
#pragma unroll
      for (int u = 0; u < U; u++)
#pragma unroll
        for (int q = 0; q < 4; q++)
          acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[u][q]),
                                                           __builtin_bit_cast(bf16x8, b[u]),
                                                           acc[q], 0, 0, 0);
    }
    // lane (r, g) holds rows 4g .. 4g+3 (experts) of column r (token)
    if (parts == 1) {
#pragma unroll
      for (int q = 0; q < 4; q++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int e = (eg * 4 + q) * 16 + 4 * g + i;
          if (vt && e < E) lgs[t * E + e] = acc[q][i];
        }
    } else {  // a single round: add the parts of each expert tile in order
#pragma unroll
      for (int q = 0; q < 4; q++) {
        if (live) {
#pragma unroll
          for (int i = 0; i < 4; i++) part[w][lane * 4 + i] = acc[q][i];
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < n_groups * 256; idx += blockDim.x) {
          const int gi = idx >> 8, l = (idx >> 2) & 63, i = idx & 3;
          float sum = 0.f;
          for (int pp = 0; pp < parts; pp++) sum += part[gi * parts + pp][l * 4 + i];
          const int e = ((gi % n_eg) * 4 + q) * 16 + 4 * (l >> 4) + i;
          const int tk = (gi / n_eg) * 16 + (l & 15);
          if (tk < T && e < E) lgs[tk * E + e] = sum;
        }
        __syncthreads();
      }
    }
  }
}

// ---------------------------------------------------------- small batches
// Exclusive scan of one int per thread over a 1024-thread block; returns the
// prefix and writes the block total to *total.  `tmp` holds 16 ints of LDS.
__device__ __forceinline__ int block_exclusive_scan_1024(int v, int* tmp, int* total) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int nb = __shfl_up(incl, o);
    if (lane >= o) incl += nb;
  }
  if (lane == kWave - 1) tmp[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    int c = tmp[i];
    if (i < w) base += c;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// The whole front of the layer for a small batch (T*k <= kRouteSmallMax
// pairs) in one block of 16 waves, so that a decode step pays one launch for
// it instead of one per stage:
//   0. with router weights wg (bf16, T * E <= kFusedRouterMaxTE, E * H <=
//      kFusedRouterMaxEH): the
//      router GEMM into LDS (router_logits_block), copied to logits_out if
//      given; the gating then reads the LDS copy;
//   1. top-k gating, one wave per token (logits == nullptr and wg ==
//      nullptr: the ids are an input instead, read from `ids`; the grouping
//      entry point runs steps 2-4 only);
//   2. expert histogram (LDS integer atomics: counts do not depend on order)
//      and its exclusive scan -> counts, offsets; thread e owns expert e;
//   3. the list of tiles of <= bm positions;
//   4. stable grouping: pair f lands at its expert's offset plus the number
//      of earlier pairs routed to the same expert, so pairs keep ascending
//      order inside each expert;
//   5. FP8 (xq != nullptr): amax(x) and the e4m3 codes of x, done by a second
//      block of the same launch, concurrently with steps 1-4 (they share no
//      data), so the two parts cost the longer of them rather than the sum.
// Every control word is written here: amax_x (block 1 in FP8 mode, else 0),
// amax_h = 0 and the tile counts (the list goes to num_tiles_big when `big`,
// the tiled GEMMs' list, else to num_tiles; the other count is 0).
__global__ __launch_bounds__(1024) void route_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm, int32_t* __restrict__ ids,
    float* __restrict__ wts, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ inv_perm, int bm, int big,
    Tile* __restrict__ tiles, Ctrl* ctrl, const uint16_t* __restrict__ x, int H,
    uint8_t* __restrict__ xq, const uint16_t* __restrict__ wg, float* __restrict__ logits_out) {
  constexpr int NW = 16;
  __shared__ __attribute__((aligned(16))) int s_ids[kRouteSmallMax];
  __shared__ __attribute__((aligned(16))) float lgs[kFusedRouterMaxTE];
  __shared__ __attribute__((aligned(16))) float rpart[NW][256];
  __shared__ __attribute__((aligned(16))) float gscr[NW][kGateScratch];
  __shared__ int hist[1024];
  __shared__ int run[1024];  // offsets of the experts
  __shared__ int tmp[NW];
  __shared__ float red[NW];
  const int t = threadIdx.x, lane = lane_id(), w = t / kWave;
  const int n = T * k;
  if (blockIdx.x == 0) {  // steps 1-4; in FP8 mode block 1 quantises x
    hist[t] = 0;

    // 0. the router GEMM into LDS
    if (wg) {
      router_logits_block(x, wg, T, H, E, lgs, rpart);
      __syncthreads();
      if (logits_out)
        for (int i = t; i < T * E; i += 1024) logits_out[i] = lgs[i];
    }
    // 1. gating (or the given ids)
    const float* lsrc = wg ? lgs : logits;
    if (lsrc) {
      for (int tok = w; tok < T; tok += NW)
        gate_token(lsrc + (size_t)tok * E, E, k, renorm, ids + (size_t)tok * k,
                   wts + (size_t)tok * k, s_ids + tok * k, gscr[w]);
    } else if (t < n) {
      s_ids[t] = ids[t];
    }
    __syncthreads();

    // 2. histogram and scans of the counts and of the tile counts
    for (int f = t; f < n; f += 1024) atomicAdd(&hist[s_ids[f]], 1);
    __syncthreads();
    const int cnt = (t < E) ? hist[t] : 0;
    const int nt = (cnt + bm - 1) / bm;
    // one scan of both counts packed in one int (each total is at most
    // kRouteSmallMax < 2^16); with E <= 64 every expert is in wave 0, whose
    // shuffle scan alone then suffices (the totals are read by thread 0)
    static_assert(kRouteSmallMax < (1 << 16), "packed scan");
    const int packed = cnt | (nt << 16);
    int ptot = 0, ppre = 0;
    if (E <= kWave) {
      if (w == 0) {
        int incl = packed;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int nb = __shfl_up(incl, o);
          if (lane >= o) incl += nb;
        }
        ppre = incl - packed;
        ptot = __shfl(incl, kWave - 1);
      }
    } else {
      ppre = block_exclusive_scan_1024(packed, tmp, &ptot);
    }
    const int pre = ppre & 0xffff, tpre = ppre >> 16;
    const int total_tiles = ptot >> 16;
    if (t < E) {
      counts[t] = cnt;
      offsets[t] = pre;
      run[t] = pre;
      // 3. tiles of this expert
      for (int i = 0; i < nt; i++) {
        Tile tl;
        tl.e = t;
        tl.p0 = pre + i * bm;
        tl.mt = min(bm, cnt - i * bm);
        tl.pad = 0;
        tiles[tpre + i] = tl;
      }
    }
    if (t == 0) offsets[E] = n;
    __syncthreads();

    // 4. stable grouping: pair f goes to its expert's offset plus the number of
    // earlier pairs on the same expert (broadcast LDS reads, no atomics)
    for (int f = t; f < n; f += 1024) {
      const int e = s_ids[f];
      int rank = 0;
      const int4* s4 = reinterpret_cast<const int4*>(s_ids);
      for (int j = 0; j < f / 4; j++) {  // 16-byte reads every lane shares
        const int4 q = s4[j];
        rank += (q.x == e) + (q.y == e) + (q.z == e) + (q.w == e);
      }
      for (int j = f & ~3; j < f; j++) rank += (s_ids[j] == e);
      const int pos = run[e] + rank;
      sorted_ids[pos] = f;
      if (inv_perm) inv_perm[f] = pos;
    }

    if (t == 0) {
      if (!xq) ctrl->amax_x_bits = 0u;
      ctrl->amax_h_bits = 0u;
      ctrl->num_tiles = big ? 0 : total_tiles;
      ctrl->num_tiles_big = big ? total_tiles : 0;
    }
  } else {
    // 5. FP8 activation quantisation (x is bf16, H a multiple of 128): four
    // 16-byte loads in flight per thread; the first four are kept in
    // registers for the encoding pass (the whole of x up to 32768 values)
    const int n8 = T * H / 8;
    const i32x4* x4 = reinterpret_cast<const i32x4*>(x);
    float m = 0.f;
    i32x4 v0[4];
    auto load4 = [&](int i0, i32x4* v) {
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int i = i0 + u * 1024;
        v[u] = (i < n8) ? x4[i] : i32x4{0, 0, 0, 0};
      }
    };
    auto amax4 = [&](const i32x4* v) {
#pragma unroll
      for (int u = 0; u < 4; u++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const uint32_t uu = (uint32_t)v[u][q];
          m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(uu & 0xffffu))));
          m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(uu >> 16))));
        }
    };
    load4(t, v0);
    amax4(v0);
    for (int i0 = t + 4 * 1024; i0 < n8; i0 += 4 * 1024) {
      i32x4 v[4];
      load4(i0, v);
      amax4(v);
    }
    m = wave_max(m);
    if (lane == 0) red[w] = m;
    __syncthreads();
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < NW; i++) a = fmaxf(a, red[i]);
    if (t == 0) ctrl->amax_x_bits = __float_as_uint(a);
    const float r = a > 0.f ? 448.0f / a : 1.0f;
    uint2* d2 = reinterpret_cast<uint2*>(xq);
    for (int i0 = t; i0 < n8; i0 += 4 * 1024) {
      i32x4 v[4];
      if (i0 == t) {
#pragma unroll
        for (int u = 0; u < 4; u++) v[u] = v0[u];
      } else {
        load4(i0, v);
      }
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int i = i0 + u * 1024;
        if (i < n8) d2[i] = bf16x8_to_e4m3x8(v[u], r);
      }
    }
  }
}

hipError_t launch_route_small(const float* logits, int T, int E, int k, int renorm, int32_t* ids,
                              float* w, int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                              int32_t* inv_perm, int bm, bool big, Tile* tiles, Ctrl* ctrl,
                              const uint16_t* x, int H, uint8_t* xq, const uint16_t* wg,
                              float* logits_out, hipStream_t st) {
  if ((long)T * k > kRouteSmallMax || E > 1024) return hipErrorInvalidValue;
  if (wg && ((long)T * E > kFusedRouterMaxTE || (long)E * H > kFusedRouterMaxEH || !x || H % 128))
    return hipErrorInvalidValue;
  route_small_kernel<<<xq ? 2 : 1, 1024, 0, st>>>(logits, T, E, k, renorm, ids, w, counts,
                                                 offsets, sorted_ids, inv_perm, bm, big ? 1 : 0,
                                                 tiles, ctrl, x, H, xq, wg, logits_out);
  return hipGetLastError();
}

// ------------------------------------------------------ large batches
// Grouping of many pairs as a counting sort over chunks of kSortChunk pairs,
// in three launches instead of one block per expert scanning every pair:
//   chunk_rank_kernel : per chunk, the expert histogram and each pair's rank
//                       among the earlier pairs of its chunk on the same
//                       expert (ballots match the lanes of a wave holding
//                       the same expert; per-wave counts are summed over
//                       the earlier waves; no atomics decide it);
//   chunk_scan_kernel : expert totals, offsets, and every chunk's starting
//                       position inside each expert's group; the tile list
//                       (and, when asked, the same tiles in the down
//                       projection's launch order);
//   chunk_scatter_kernel : position = chunk base of the expert + rank.
// Positions are therefore ordered by (expert, pair index), the same stable
// order as the one-kernel grouping.
__global__ __launch_bounds__(1024) void chunk_rank_kernel(const int32_t* __restrict__ ids, int n,
                                                          int E, int32_t* __restrict__ chunk_counts,
                                                          int32_t* __restrict__ rank,
                                                          int n_chunks, XWork xw) {
  constexpr int NW = kSortChunk / kWave;  // waves of the block, one pair per thread
  __shared__ int whist[NW][1024];         // pairs of wave w on expert e
  if ((int)blockIdx.x >= n_chunks) {  // block-uniform: the x encoding blocks
    x_quant_part(xw, blockIdx.x - n_chunks, kXQuantBlocks);
    return;
  }
  const int t = threadIdx.x, c = blockIdx.x, w = t / kWave, lane = lane_id();
  const int f0 = c * kSortChunk, m = min(kSortChunk, n - f0);
  for (int i = t; i < NW * E; i += blockDim.x) whist[i / E][i % E] = 0;
  const bool valid = t < m;
  const int e = valid ? ids[f0 + t] : 0;
  // lanes of this wave holding the same expert: one ballot per bit of the
  // expert index (E <= 1024: ten bits), narrowed to the valid lanes
  uint64_t same = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 10; b++) {
    const bool bit = (e >> b) & 1;
    const uint64_t ones = __ballot(bit);
    same &= bit ? ones : ~ones;
  }
  const int intra = __popcll(same & ((1ull << lane) - 1));  // earlier lanes, same expert
  __syncthreads();  // whist zeroed
  // the first lane of each expert group records the group's size (one
  // writer per (wave, expert): no atomics)
  if (valid && intra == 0) whist[w][e] = __popcll(same);
  __syncthreads();
  // rank = pairs of earlier waves on the expert + earlier lanes of this wave
  if (valid) {
    int r = intra;
    for (int i = 0; i < w; i++) r += whist[i][e];
    rank[f0 + t] = r;
  }
  for (int ee = t; ee < E; ee += blockDim.x) {
    int s = 0;
#pragma unroll
    for (int i = 0; i < NW; i++) s += whist[i][ee];
    chunk_counts[(size_t)c * E + ee] = s;
  }
}

// The spread order of n tiles, F of them full: full tile a (counted in list
// order) goes to position a * n / F, and the partial tiles fill the positions
// left, in list order: partial tile b takes the smallest p at which the count
// of free positions up to p, p + 1 - ceil((p + 1) F / n), reaches b + 1.  A
// permutation of 0 .. n-1.
// U is the integer type of the products: 32-bit while n * n fits (a 64-bit
// division is a long software routine, and one thread per expert places all
// of its expert's tiles).
template <typename U>
__device__ __forceinline__ int partial_position(int rank, int n, int F) {
  int lo = rank, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const U q = (U)(mid + 1);
    if (q - (q * (U)F + (U)(n - 1)) / (U)n >= (U)(rank + 1))
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

// Writes one expert's tiles (nfull full ones, then at most one partial one,
// the first full one of list rank a0, the partial one of rank b) at their
// spread positions; successive full positions a * n / F advance by n / F
// with a carry, so the loop divides nothing.
template <typename U>
__device__ __forceinline__ void place_spread(Tile tl, int bm, int cnt, int nfull, int a0, int b,
                                             int n, int F, Tile* __restrict__ out) {
  if (nfull > 0) {
    const U step_q = (U)n / (U)F, step_r = (U)n % (U)F;
    U q = (U)a0 * (U)n / (U)F, rem = (U)a0 * (U)n % (U)F;
    for (int i = 0; i < nfull; i++) {
      tl.p0 = tl.p0 + (i ? bm : 0);
      tl.mt = bm;
      out[(int)q] = tl;
      q += step_q;
      rem += step_r;
      if (rem >= (U)F) rem -= (U)F, q += 1;
    }
  }
  if (cnt > nfull * bm) {
    tl.p0 = tl.p0 + (nfull ? bm : 0);
    tl.mt = cnt - nfull * bm;
    out[partial_position<U>(b, n, F)] = tl;
  }
}

__global__ __launch_bounds__(1024) void chunk_scan_kernel(
    const int32_t* __restrict__ chunk_counts, int n_chunks, int E, int n,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ base,
    int bm, Tile* __restrict__ tiles, int32_t* num_tiles, Tile* __restrict__ tiles_spread) {
  __shared__ int tmp[16];
  const int t = threadIdx.x;
  int cnt = 0;
  // the column of chunk counts of expert t, eight independent loads in
  // flight at a time (one at a time left this kernel latency-bound: 14 us at
  // 32 chunks, 47 us at 128)
  if (t < E) {
    int c = 0;
    for (; c + 8 <= n_chunks; c += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; u++) v[u] = chunk_counts[(size_t)(c + u) * E + t];
#pragma unroll
      for (int u = 0; u < 8; u++) cnt += v[u];
    }
    for (; c < n_chunks; c++) cnt += chunk_counts[(size_t)c * E + t];
  }
  const int nt = (cnt + bm - 1) / bm;
  const int nfull = cnt / bm;  // tiles of exactly bm positions, listed first
  int total_pairs, total_tiles, total_full = 0;
  const int pre = block_exclusive_scan_1024(cnt, tmp, &total_pairs);
  const int tpre = block_exclusive_scan_1024(nt, tmp, &total_tiles);
  int fpre = 0;
  if (tiles_spread) fpre = block_exclusive_scan_1024(nfull, tmp, &total_full);
  if (t < E) {
    counts[t] = cnt;
    offsets[t] = pre;
    int run = pre;
    int c = 0;
    for (; c + 8 <= n_chunks; c += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; u++) v[u] = chunk_counts[(size_t)(c + u) * E + t];
#pragma unroll
      for (int u = 0; u < 8; u++) {
        base[(size_t)(c + u) * E + t] = run;
        run += v[u];
      }
    }
    for (; c < n_chunks; c++) {
      base[(size_t)c * E + t] = run;
      run += chunk_counts[(size_t)c * E + t];
    }
    for (int i = 0; i < nt; i++) {
      Tile tl;
      tl.e = t;
      tl.p0 = pre + i * bm;
      tl.mt = min(bm, cnt - i * bm);
      tl.pad = 0;
      tiles[tpre + i] = tl;
    }
    if (tiles_spread && nt > 0) {
      // list ranks: this expert's full tiles follow fpre full ones, its
      // partial tile follows the tpre - fpre partial ones before it
      const Tile first = {t, pre, 0, 0};
      if (total_tiles <= 65535)
        place_spread<uint32_t>(first, bm, cnt, nfull, fpre, tpre - fpre, total_tiles, total_full,
                               tiles_spread);
      else
        place_spread<uint64_t>(first, bm, cnt, nfull, fpre, tpre - fpre, total_tiles, total_full,
                               tiles_spread);
    }
  }
  if (t == 0) {
    offsets[E] = n;
    *num_tiles = total_tiles;
  }
}

__global__ __launch_bounds__(1024) void chunk_scatter_kernel(const int32_t* __restrict__ ids,
                                                             const int32_t* __restrict__ rank,
                                                             const int32_t* __restrict__ base,
                                                             int n, int E,
                                                             int32_t* __restrict__ sorted_ids,
                                                             int32_t* __restrict__ inv_perm) {
  const int f = blockIdx.x * 1024 + threadIdx.x;
  if (f >= n) return;
  const int pos = base[(size_t)(f / kSortChunk) * E + ids[f]] + rank[f];
  sorted_ids[pos] = f;
  inv_perm[f] = pos;
}

hipError_t launch_chunk_sort(const int32_t* ids, int n, int E, int32_t* counts, int32_t* offsets,
                             int32_t* sorted_ids, int32_t* inv_perm, int bm, Tile* tiles,
                             int32_t* num_tiles, int32_t* chunk_counts, int32_t* base,
                             int32_t* rank, hipStream_t st, const XWork* xw,
                             Tile* tiles_spread) {
  const int n_chunks = (n + kSortChunk - 1) / kSortChunk;
  chunk_rank_kernel<<<n_chunks + (xw ? kXQuantBlocks : 0), 1024, 0, st>>>(
      ids, n, E, chunk_counts, rank, n_chunks, xw ? *xw : XWork{});
  chunk_scan_kernel<<<1, 1024, 0, st>>>(chunk_counts, n_chunks, E, n, counts, offsets, base, bm,
                                        tiles, num_tiles, tiles_spread);
  chunk_scatter_kernel<<<(n + 1023) / 1024, 1024, 0, st>>>(ids, rank, base, n, E, sorted_ids,
                                                           inv_perm);
  return hipGetLastError();
}

}  // namespace moe
