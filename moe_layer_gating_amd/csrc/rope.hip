// rope.hip -- inverse rotary position embedding fused with per-head FP8
// quantisation, over a token count that is a runtime argument.
//
// The pages' second fused kernel: a rotary-embedding plus FP8-quantisation
// kernel whose token count changes from call to call, and which a JIT
// rebuilt for every new count until its variable-length parameters stopped
// being specialisation keys (codebridge-ai.com, "aws-moe-kernel-wgmma-triton-
// ttft", section "3. Kill JIT recompilation"; agentic-affairs.com, "Removing
// recompilation improves the first-token result").  Here the kernel is
// compiled once, ahead of time, and T, the head count and the positions are
// plain arguments read at run time.
//
// For token t (position p = positions[t], clamped into the table) and each
// head, over the first rot_dim values, a coordinate pair (a, b) with table
// cosine c and sine s (row p of cos_sin: rot_dim/2 cosines, then the sines)
// becomes
//     y_a = x_a c + x_b s,     y_b = x_b c - x_a s
// (the rotation by the negative angle), pairs being (i, i + rot_dim/2) or,
// interleaved, (2i, 2i+1); values past rot_dim pass through.  Each product
// and each sum is one fp32 operation (no fused multiply-add), because the
// e4m3 codes are decided on y.  The head is then quantised with its own
// dynamic scale: A = max |y| over the head, scale = fl32(A / 448), codes
// e4m3(fl32(y * fl32(448 / A))), A = 0 giving scale 1.
//
// Memory traffic is one read of x, one write of the codes and scales, and
// the table rows of the batch's positions.
#include "moe_common.h"

namespace moe {

// Rotate-half pairing: a head's work units are its rot_dim/16 chunk pairs
// (chunk u with chunk u + rot_dim/16: the pairs (8u + j, 8u + j +
// rot_dim/2), j < 8) and its (head_dim - rot_dim)/8 pass-through chunks; one
// thread per unit, so each value and each table entry is loaded once.
// Interleaved pairing: one thread per chunk (its pairs lie inside it).  A
// head's units occupy G = next power of two lanes, so its amax is a
// butterfly over G lanes.  A thread takes the same unit of HPT consecutive
// heads of one token (HPT divides the head count): the token's table entries
// are loaded once for all of them, and HPT heads' loads are in flight.
template <bool INTER, int HPT>
__global__ __launch_bounds__(256) void inv_rope_fp8_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ positions,
    const float* __restrict__ cos_sin, long n_heads_total, int n_heads, int head_dim, int rot_dim,
    int max_pos, int G, uint8_t* __restrict__ codes, float* __restrict__ scales) {
  // each product and each sum rounded on its own: no multiply-add fusion.
  // hipcc contracts by default; this pragma governs the operators written
  // in this body (not those inside header functions such as __fadd_rn,
  // which keep the default), so the arithmetic below uses plain operators.
#pragma clang fp contract(off)
  const int lane = lane_id();
  const int u = lane & (G - 1);  // work unit of the head
  const long hg = ((long)blockIdx.x * blockDim.x + threadIdx.x) / G;  // group of HPT heads
  const int half = rot_dim / 2;
  const int h8 = rot_dim / 16;  // chunk pairs (rotate half)
  const int units = INTER ? head_dim / 8 : h8 + (head_dim - rot_dim) / 8;
  const bool live = hg * HPT < n_heads_total && u < units;
  // chunk c0 holds y[0..8); rotate-half pair units also chunk c1 = c0 + h8
  // with y[8..16)
  const int c0 = INTER || u < h8 ? u : u + h8;
  const bool pair = !INTER && u < h8;
  float y[HPT][16];
  float m[HPT];
#pragma unroll
  for (int hh = 0; hh < HPT; hh++) m[hh] = 0.f;
  if (live) {
    const long th0 = hg * HPT;
    const long t = th0 / n_heads;
    int p = positions[t];
    p = p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
    const float* cs = cos_sin + (size_t)p * rot_dim;
    // the unit's table entries: cosines then sines of its 4 (interleaved)
    // or 8 (rotate half) pairs
    float cv[8], sv[8];
    if (INTER) {
      if (8 * c0 < rot_dim) {
        const f32x4 c = *reinterpret_cast<const f32x4*>(cs + 4 * c0);
        const f32x4 s = *reinterpret_cast<const f32x4*>(cs + half + 4 * c0);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          cv[j] = c[j];
          sv[j] = s[j];
        }
      }
    } else if (pair) {
      const f32x4 ca = *reinterpret_cast<const f32x4*>(cs + 8 * c0);
      const f32x4 cb = *reinterpret_cast<const f32x4*>(cs + 8 * c0 + 4);
      const f32x4 sa = *reinterpret_cast<const f32x4*>(cs + half + 8 * c0);
      const f32x4 sb = *reinterpret_cast<const f32x4*>(cs + half + 8 * c0 + 4);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        cv[j] = ca[j];
        cv[4 + j] = cb[j];
        sv[j] = sa[j];
        sv[4 + j] = sb[j];
      }
    }
    i32x4 v0[HPT], v1[HPT];
#pragma unroll
    for (int hh = 0; hh < HPT; hh++) {
      const uint16_t* xh = x + (size_t)(th0 + hh) * head_dim;
      v0[hh] = *reinterpret_cast<const i32x4*>(xh + 8 * c0);
      if (pair) v1[hh] = *reinterpret_cast<const i32x4*>(xh + 8 * (c0 + h8));
    }
#pragma unroll
    for (int hh = 0; hh < HPT; hh++) {
      float* yh = y[hh];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        yh[2 * j] = bf16_to_f32((uint16_t)((uint32_t)v0[hh][j] & 0xffffu));
        yh[2 * j + 1] = bf16_to_f32((uint16_t)((uint32_t)v0[hh][j] >> 16));
        if (pair) {
          yh[8 + 2 * j] = bf16_to_f32((uint16_t)((uint32_t)v1[hh][j] & 0xffffu));
          yh[8 + 2 * j + 1] = bf16_to_f32((uint16_t)((uint32_t)v1[hh][j] >> 16));
        }
      }
      if (INTER) {
        if (8 * c0 < rot_dim) {  // pairs (2i, 2i+1), i = 4 c0 + j
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const float xa = yh[2 * j], xb = yh[2 * j + 1];
            yh[2 * j] = xa * cv[j] + xb * sv[j];
            yh[2 * j + 1] = xb * cv[j] - xa * sv[j];
          }
        }
      } else if (pair) {  // pairs (8 c0 + j, 8 c0 + j + half)
#pragma unroll
        for (int j = 0; j < 8; j++) {
          const float xa = yh[j], xb = yh[8 + j];
          yh[j] = xa * cv[j] + xb * sv[j];
          yh[8 + j] = xb * cv[j] - xa * sv[j];
        }
      }
#pragma unroll
      for (int j = 0; j < 16; j++)
        if (j < 8 || pair) m[hh] = fmaxf(m[hh], fabsf(yh[j]));
    }
  }
  // amax over each head's G lanes (G divides 64; groups are lane-aligned)
#pragma unroll
  for (int hh = 0; hh < HPT; hh++)
    for (int o = 1; o < G; o <<= 1) m[hh] = fmaxf(m[hh], __shfl_xor(m[hh], o));
  if (!live) return;
#pragma unroll
  for (int hh = 0; hh < HPT; hh++) {
    const long th = hg * HPT + hh;
    const float sc = m[hh] > 0.f ? m[hh] / 448.0f : 1.0f;
    const float r = m[hh] > 0.f ? 448.0f / m[hh] : 1.0f;
    uint8_t* ch = codes + (size_t)th * head_dim;
#pragma unroll
    for (int k8 = 0; k8 < 2; k8++) {
      if (k8 == 1 && !pair) break;
      float f[8];
#pragma unroll
      for (int j = 0; j < 8; j++)
        f[j] = __builtin_amdgcn_fmed3f(y[hh][8 * k8 + j] * r, -448.0f, 448.0f);
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
      *reinterpret_cast<uint2*>(ch + 8 * (c0 + k8 * h8)) = make_uint2((uint32_t)lo, (uint32_t)hi);
    }
    if (u == 0) scales[th] = sc;
  }
}

// Heads per thread: 4 when the head count allows it and the batch still
// gives every CU several blocks, else 1.
constexpr long kRopeMultiHeadMin = 16384;  // heads

hipError_t launch_inv_rope_fp8(const uint16_t* x, const int32_t* positions, const float* cos_sin,
                               int T, int n_heads, int head_dim, int rot_dim, int max_pos,
                               bool interleaved, uint8_t* codes, float* scales, hipStream_t st) {
  const int units = interleaved ? head_dim / 8 : rot_dim / 16 + (head_dim - rot_dim) / 8;
  int G = 1;
  while (G < units) G <<= 1;
  if (G > kWave) return hipErrorInvalidValue;
  const long heads = (long)T * n_heads;
  const int hpt = (n_heads % 4 == 0 && heads >= kRopeMultiHeadMin) ? 4 : 1;
  const long threads = heads / hpt * G;
  const long grid = (threads + 255) / 256;
  if (grid <= 0) return hipSuccess;
#define MOE_ROPE(INTER_, HPT_)                                                              \
  inv_rope_fp8_kernel<INTER_, HPT_><<<grid, 256, 0, st>>>(x, positions, cos_sin, heads, n_heads, \
                                                          head_dim, rot_dim, max_pos, G, codes,  \
                                                          scales)
  if (interleaved) {
    if (hpt == 4)
      MOE_ROPE(true, 4);
    else
      MOE_ROPE(true, 1);
  } else {
    if (hpt == 4)
      MOE_ROPE(false, 4);
    else
      MOE_ROPE(false, 1);
  }
#undef MOE_ROPE
  return hipGetLastError();
}

}  // namespace moe
