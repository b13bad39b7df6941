// Device helpers shared by the decode and chunk kernels: weight-code
// conversion to binary16, packed dot products, wave reductions and the
// agent-scope counters used between workgroups of one launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_w4a16.h"

namespace moe {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

static constexpr int kGroup = 64;     // quantisation group along K
static constexpr int kMaxTopK = 8;
static constexpr int kMaxExperts = 256;

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// ---------------------------------------------------------------------------
// Weight codes -> exact binary16 integers.
//
// Both conversions return the eight codes of two 32-bit words in the order
// (k0,k4), (k1,k5), (k2,k6), (k3,k7): element i of the 8-vector is
// K offset perm8(i) = {0,4,1,5,2,6,3,7}[i].  Activations are permuted the same
// way, so every dot product sees matching pairs.
//
// The conversion ORs a biased code into the mantissa of a binary16 constant
// (1024 has unit spacing, 64 has spacing 1/16) and subtracts the constant and
// the bias, which is exact.
// ---------------------------------------------------------------------------

// mask ? (x ^ b) : b, bit by bit (a single v_bitop3 on gfx950).  With b
// holding the sign bit of each field under the mask and the binary16 constant
// outside it, this turns two's complement fields into biased codes and ORs
// them into the constant in one instruction.
__device__ __forceinline__ uint32_t flip_into(uint32_t x, uint32_t mask, uint32_t b) {
  return (mask & (x ^ b)) | (~mask & b);
}

// one word = 8 int4 codes (k0 in bits 0-3 ... k7 in bits 28-31)
__device__ __forceinline__ void int4x8_to_h2x4(uint32_t w, h2 out[4]) {
  const uint32_t v = w >> 8;
  const h2 lo_bias = as_h2(0x64086408u);  // 1032 = 1024 + 8
  const h2 hi_bias = as_h2(0x54805480u);  // 72 = 64 + 8
  out[0] = as_h2(flip_into(w, 0x000F000Fu, 0x64086408u)) - lo_bias;  // (k0, k4)
  out[1] = as_h2(flip_into(w, 0x00F000F0u, 0x54805480u)) - hi_bias;  // (k1, k5)
  out[2] = as_h2(flip_into(v, 0x000F000Fu, 0x64086408u)) - lo_bias;  // (k2, k6)
  out[3] = as_h2(flip_into(v, 0x00F000F0u, 0x54805480u)) - hi_bias;  // (k3, k7)
}

// one word = 8 UNSIGNED 4-bit codes (affine int4), same output order: each
// field is ORed into the mantissa of 1024 (unit spacing) or 64 (spacing 1/16)
// and the constant subtracted, which is exact
__device__ __forceinline__ void uint4x8_to_h2x4(uint32_t w, h2 out[4]) {
  const uint32_t v = w >> 8;
  const h2 lo_c = as_h2(0x64006400u);  // 1024
  const h2 hi_c = as_h2(0x54005400u);  // 64
  out[0] = as_h2((w & 0x000F000Fu) | 0x64006400u) - lo_c;  // (k0, k4)
  out[1] = as_h2((w & 0x00F000F0u) | 0x54005400u) - hi_c;  // (k1, k5)
  out[2] = as_h2((v & 0x000F000Fu) | 0x64006400u) - lo_c;  // (k2, k6)
  out[3] = as_h2((v & 0x00F000F0u) | 0x54005400u) - hi_c;  // (k3, k7)
}

// two words = 8 int8 codes (w0: k0..k3, w1: k4..k7), same output order
__device__ __forceinline__ void int8x8_to_h2x4(uint32_t w0, uint32_t w1, h2 out[4]) {
  const uint32_t a = __builtin_amdgcn_perm(w1, w0, 0x05040100u);  // k0 k1 k4 k5
  const uint32_t b = __builtin_amdgcn_perm(w1, w0, 0x07060302u);  // k2 k3 k6 k7
  const h2 bias = as_h2(0x64806480u);  // 1152 = 1024 + 128
  out[0] = as_h2(flip_into(a, 0x00FF00FFu, 0x64806480u)) - bias;       // (k0, k4)
  out[1] = as_h2(flip_into(a >> 8, 0x00FF00FFu, 0x64806480u)) - bias;  // (k1, k5)
  out[2] = as_h2(flip_into(b, 0x00FF00FFu, 0x64806480u)) - bias;       // (k2, k6)
  out[3] = as_h2(flip_into(b >> 8, 0x00FF00FFu, 0x64806480u)) - bias;  // (k3, k7)
}

// Eight activations in natural order (4 words: [x1:x0] [x3:x2] [x5:x4] [x7:x6])
// -> the pair order used above.
__device__ __forceinline__ void perm8_words(const uint32_t x[4], uint32_t out[4]) {
  out[0] = __builtin_amdgcn_perm(x[2], x[0], 0x05040100u);  // (x0, x4)
  out[1] = __builtin_amdgcn_perm(x[2], x[0], 0x07060302u);  // (x1, x5)
  out[2] = __builtin_amdgcn_perm(x[3], x[1], 0x05040100u);  // (x2, x6)
  out[3] = __builtin_amdgcn_perm(x[3], x[1], 0x07060302u);  // (x3, x7)
}

__device__ __forceinline__ float dot2(h2 a, h2 b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}

// z sigmoid(z) with the hardware reciprocal (about 1 ulp) in place of an IEEE
// division: the result is rounded to binary16 where it is used
__device__ __forceinline__ float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + expf(-z)); }

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// ---------------------------------------------------------------------------
// wave-level reductions (wave64)
// ---------------------------------------------------------------------------

// butterfly sum within aligned groups of `width` lanes (power of two <= 64)
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int m = 1; m < width; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// DPP helpers: quad_perm(1,0,3,2), quad_perm(2,3,0,1), row_ror 4, row_ror 8
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

// maximum over all 64 lanes, returned uniformly
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x124>(v));
  v = max(v, dpp_u32<0x128>(v));
  uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return ~wave_max_u32(~v);
}

// float -> unsigned key with the same order (-0 folded onto +0)
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __builtin_bit_cast(float, u);
}

// Sums within aligned groups of `width` lanes (power of two <= 64); every lane
// of a group receives the group's sum.  Rows of 16 lanes reduce with DPP.
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dppf<0xB1>(v);   // quad_perm(1,0,3,2)
  v += dppf<0x4E>(v);   // quad_perm(2,3,0,1)
  v += dppf<0x124>(v);  // row_ror 4
  v += dppf<0x128>(v);  // row_ror 8
  return v;
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float lane_group_sum(float v, int width) {
  if (width == 64) {
    v = row16_sum(v);
    return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
  }
  if (width == 32) {
    v = row16_sum(v);
    return v + __shfl_xor(v, 16, 64);
  }
  if (width == 16) return row16_sum(v);
  for (int m = 1; m < width; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// ---------------------------------------------------------------------------
// top-k
// ---------------------------------------------------------------------------

struct TopkScratch {
  uint64_t comp[kMaxExperts];  // candidates: (order key << 32) | (0xFFFF - expert)
  int sel_idx[kMaxTopK];
  float sel_val[kMaxTopK];
};

// Top-k of one token's E router logits by ONE wave, with no workgroup
// barrier.  Lane l holds the logits of experts 4l .. 4l+3 in v[] (entries at
// or past E are ignored).
//
// Selection is by logit (softmax is monotone), descending, ties to the lower
// expert index; the kept probabilities are renormalised, which equals a
// softmax over the k kept logits.  With at least k groups of 32 experts, the
// smallest group maximum tau bounds the k-th largest logit from below, so
// only the experts at or above tau are candidates.  Candidates are compacted
// by ballot and ranked, each against every other, on a 64-bit key that orders
// by (logit desc, expert asc) and is unique.  Lanes 0..k-1 write ids_out and
// w_out (rank order).
__device__ inline void wave_topk(const float v[4], int E, int k, int* ids_out, float* w_out, TopkScratch& sc) {
  const int lane = threadIdx.x & 63;
  uint32_t key[4];
  bool ok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ok[j] = 4 * lane + j < E;
    key[j] = ok[j] ? order_key(v[j]) : 0u;
  }
  uint32_t tau = 0;
  if ((E + 31) / 32 >= k) {  // uniform
    // maximum of each 32-expert group (8 lanes), spread over its lanes
    uint32_t m = max(max(key[0], key[1]), max(key[2], key[3]));
    m = max(m, dpp_u32<0xB1>(m));  // quad_perm(1,0,3,2)
    m = max(m, dpp_u32<0x4E>(m));  // quad_perm(2,3,0,1)
    m = max(m, (uint32_t)__shfl_xor((int)m, 4, 64));
    // smallest maximum over the groups that hold experts
    tau = wave_min_u32(4 * lane < E ? m : 0xFFFFFFFFu);
  }
  int base = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool cand = ok[j] && key[j] >= tau;
    const uint64_t bal = __ballot(cand);
    const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (cand) sc.comp[pos] = ((uint64_t)key[j] << 32) | (uint64_t)(0xFFFFu - (uint32_t)(4 * lane + j));
    base += __popcll(bal);
  }
  const int C = base;
  __builtin_amdgcn_wave_barrier();
  for (int c0 = lane; c0 < C; c0 += 64) {
    const uint64_t my = sc.comp[c0];
    int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
    int c = 0;
    for (; c + 3 < C; c += 4) {
      r0 += sc.comp[c] > my;
      r1 += sc.comp[c + 1] > my;
      r2 += sc.comp[c + 2] > my;
      r3 += sc.comp[c + 3] > my;
    }
    for (; c < C; ++c) r0 += sc.comp[c] > my;
    const int rank = (r0 + r1) + (r2 + r3);
    if (rank < k) {
      sc.sel_idx[rank] = (int)(0xFFFFu - (uint32_t)(my & 0xFFFFu));
      sc.sel_val[rank] = key_to_float((uint32_t)(my >> 32));
    }
  }
  __builtin_amdgcn_wave_barrier();
  const float v0 = sc.sel_val[0];
  const float e = lane < k ? expf(sc.sel_val[lane < k ? lane : 0] - v0) : 0.f;
  const float s = row16_sum(e);  // k <= 8: lanes 0..k-1 sit in row 0
  if (lane < k) {
    ids_out[lane] = sc.sel_idx[lane];
    w_out[lane] = e / s;
  }
}

}  // namespace moe
