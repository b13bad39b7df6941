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

// one word = 8 int4 codes (k0 in bits 0-3 ... k7 in bits 28-31)
__device__ __forceinline__ void int4x8_to_h2x4(uint32_t w, h2 out[4]) {
  const uint32_t u = w ^ 0x88888888u;  // two's complement -> code + 8 in [0, 15]
  const uint32_t v = u >> 8;
  const h2 lo_bias = as_h2(0x64086408u);  // 1032 = 1024 + 8
  const h2 hi_bias = as_h2(0x54805480u);  // 72 = 64 + 8
  out[0] = as_h2((u & 0x000F000Fu) | 0x64006400u) - lo_bias;  // (k0, k4)
  out[1] = as_h2((u & 0x00F000F0u) | 0x54005400u) - hi_bias;  // (k1, k5)
  out[2] = as_h2((v & 0x000F000Fu) | 0x64006400u) - lo_bias;  // (k2, k6)
  out[3] = as_h2((v & 0x00F000F0u) | 0x54005400u) - hi_bias;  // (k3, k7)
}

// two words = 8 int8 codes (w0: k0..k3, w1: k4..k7), same output order
__device__ __forceinline__ void int8x8_to_h2x4(uint32_t w0, uint32_t w1, h2 out[4]) {
  const uint32_t a = __builtin_amdgcn_perm(w1, w0, 0x05040100u) ^ 0x80808080u;  // k0 k1 k4 k5 (+128)
  const uint32_t b = __builtin_amdgcn_perm(w1, w0, 0x07060302u) ^ 0x80808080u;  // k2 k3 k6 k7 (+128)
  const h2 bias = as_h2(0x64806480u);  // 1152 = 1024 + 128
  out[0] = as_h2((a & 0x00FF00FFu) | 0x64006400u) - bias;         // (k0, k4)
  out[1] = as_h2(((a >> 8) & 0x00FF00FFu) | 0x64006400u) - bias;  // (k1, k5)
  out[2] = as_h2((b & 0x00FF00FFu) | 0x64006400u) - bias;         // (k2, k6)
  out[3] = as_h2(((b >> 8) & 0x00FF00FFu) | 0x64006400u) - bias;  // (k3, k7)
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

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }
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

// ---------------------------------------------------------------------------
// Top-k of one token's router logits by one wave.
//
// Selection is by logit (softmax is monotone), descending, ties to the lower
// expert index; the kept probabilities are renormalised, which equals a
// softmax over the k kept logits.  Results are uniform across the wave.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void wave_topk(const float* logits, int E, int k, int* ids, float* w) {
  const int lane = threadIdx.x & 63;
  uint32_t key[4];
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    key[j] = (e < E) ? order_key(logits[e]) : 0u;
  }
  uint32_t removed = 0;  // bit j: element lane + 64 j already taken
  float val[kMaxTopK];
  for (int r = 0; r < k; ++r) {
    uint32_t best = 0;
    int bj = -1;
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e < E && !((removed >> j) & 1u) && (bj < 0 || key[j] > best)) { best = key[j]; bj = j; }
    }
    const uint32_t m = wave_max_u32(bj >= 0 ? best : 0u);
    const uint64_t hit = __ballot(bj >= 0 && best == m);
    int win;
    if (__popcll(hit) == 1) {
      const int wl = __ffsll((unsigned long long)hit) - 1;
      const int wj = __shfl(bj, wl, 64);
      win = wl + 64 * wj;
    } else {
      const uint32_t mine = (bj >= 0 && best == m) ? (uint32_t)(lane + 64 * bj) : 0xFFFFFFFFu;
      win = (int)wave_min_u32(mine);
    }
    if (lane == (win & 63)) removed |= 1u << (win >> 6);
    ids[r] = win;
    val[r] = key_to_float(m);
  }
  float s = 0.f;
  for (int r = 0; r < k; ++r) { w[r] = expf(val[r] - val[0]); s += w[r]; }
  const float inv = 1.0f / s;
  for (int r = 0; r < k; ++r) w[r] *= inv;
}

// ---------------------------------------------------------------------------
// Counters shared by the workgroups of one persistent launch.  Producers make
// their stores visible at agent scope before counting; consumers acquire.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void signal_add(uint32_t* ctr, uint32_t v) {
  __hip_atomic_fetch_add(ctr, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t acquire_load(uint32_t* ctr) {
  return __hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace moe
