// Wave-level dequant-in-register GEMV pieces for few-token (decode) work.
//
// A weight row of K codes is split into 16-byte chunks (32 int4 or 16 int8
// codes).  With CPR = K*bits/128 chunks per row, a wave covers one row per
// load when CPR >= 64 (each lane then owns CPR/64 chunks of every row) and
// 64/CPR rows per load otherwise (groups of CPR lanes per row).  Every load is
// a coalesced 128-bit load of packed codes; activations come from LDS.
#pragma once
#include "common.hpp"

namespace moe {

struct RowGeom {
  int lpr;  // lanes per row (power of two, <= 64)
  int rpb;  // rows per wave-load (64 / lpr)
  int cpl;  // chunks per lane per row
  int cpr;  // chunks per row
};

__device__ __forceinline__ RowGeom row_geom(int K, int bits) {
  RowGeom g;
  g.cpr = K * bits / 128;
  g.lpr = g.cpr < 64 ? g.cpr : 64;
  g.rpb = 64 / g.lpr;
  g.cpl = g.cpr / g.lpr;
  return g;
}

// 32 activations (one int4 chunk) from LDS, as 16 permuted pairs
__device__ __forceinline__ void act32(const _Float16* a, h2 xp[16]) {
  const uint4* p = reinterpret_cast<const uint4*>(a);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = p[q];
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
    perm8_words(x, o);
#pragma unroll
    for (int i = 0; i < 4; ++i) xp[4 * q + i] = as_h2(o[i]);
  }
}

// 16 activations (one int8 chunk) from LDS, as 8 permuted pairs
__device__ __forceinline__ void act16(const _Float16* a, h2 xp[8]) {
  const uint4* p = reinterpret_cast<const uint4*>(a);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint4 v = p[q];
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
    perm8_words(x, o);
#pragma unroll
    for (int i = 0; i < 4; ++i) xp[4 * q + i] = as_h2(o[i]);
  }
}

// sum over one chunk of (code * activation); codes are exact integers
__device__ __forceinline__ float chunk_dot4(uint4 wq, const h2 xp[16]) {
  const uint32_t ws[4] = {wq.x, wq.y, wq.z, wq.w};
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    h2 w[4];
    int4x8_to_h2x4(ws[q], w);
#pragma unroll
    for (int p = 0; p < 4; ++p) acc = dot2(w[p], xp[4 * q + p], acc);
  }
  return acc;
}

// the same for unsigned codes (affine int4)
__device__ __forceinline__ float chunk_dot4u(uint4 wq, const h2 xp[16]) {
  const uint32_t ws[4] = {wq.x, wq.y, wq.z, wq.w};
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    h2 w[4];
    uint4x8_to_h2x4(ws[q], w);
#pragma unroll
    for (int p = 0; p < 4; ++p) acc = dot2(w[p], xp[4 * q + p], acc);
  }
  return acc;
}

__device__ __forceinline__ float chunk_dot8(uint4 wq, const h2 xp[8]) {
  float acc = 0.f;
  h2 w[4];
  int8x8_to_h2x4(wq.x, wq.y, w);
#pragma unroll
  for (int p = 0; p < 4; ++p) acc = dot2(w[p], xp[p], acc);
  int8x8_to_h2x4(wq.z, wq.w, w);
#pragma unroll
  for (int p = 0; p < 4; ++p) acc = dot2(w[p], xp[4 + p], acc);
  return acc;
}

// Group index of chunk c: int4 chunks hold 32 codes (two per group), int8
// chunks hold 16 codes (four per group).
template <int BITS>
__device__ __forceinline__ int chunk_group(int c) { return BITS == 4 ? (c >> 1) : (c >> 2); }

// per-lane 16-byte chunks of up to NB row-batches.  AFF (int4 only): the codes
// are unsigned and each group also has a binary16 offset b, so a chunk adds
// s * (q . x) + b * (sum of the chunk's 32 activations); the chunk sums of an
// activation vector come from the caller (xs, one float per 32 elements).
template <int BITS, int NB, int MAXCPL, bool AFF = false>
struct Frag {
  uint4 q[NB][MAXCPL];
  uint16_t s[NB][MAXCPL];  // binary16 scale bits (converted where they are used)
  uint16_t o[NB][MAXCPL];  // AFF: binary16 offset bits

  // rows[b]: this lane's row pointer in batch b (nullptr = masked); srow: its
  // scales (always a valid row).  A masked lane reads `safe` (a valid row)
  // instead: its products land in its own row's accumulator, which the caller
  // discards.  Only pointers are selected, never loaded values, so every load
  // of the batch is in flight before the first one is waited for.
  __device__ __forceinline__ void load(const uint8_t* const rows[NB], const uint16_t* const srow[NB],
                                       const RowGeom& g, const uint8_t* safe) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int m = 0; m < MAXCPL; ++m) {
        const int c = (lane % g.lpr) + g.lpr * (m < g.cpl ? m : 0);
        const uint8_t* src = rows[b] != nullptr ? rows[b] : safe;
        q[b][m] = *reinterpret_cast<const uint4*>(src + 16 * (size_t)c);
        s[b][m] = srow[b][chunk_group<BITS>(c)];
      }
  }

  // AFF: the offsets, same indexing as the scales (orow[b] a valid row)
  __device__ __forceinline__ void load_offsets(const uint16_t* const orow[NB], const RowGeom& g) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int m = 0; m < MAXCPL; ++m) {
        const int c = (lane % g.lpr) + g.lpr * (m < g.cpl ? m : 0);
        o[b][m] = orow[b][chunk_group<BITS>(c)];
      }
  }

  __device__ __forceinline__ float chunk4(uint4 wq, const h2 xp[16], uint16_t sb, uint16_t ob, float xsum,
                                          float acc) const {
    if (AFF) {
      acc = fmaf(chunk_dot4u(wq, xp), half_bits_to_float(sb), acc);
      return fmaf(xsum, half_bits_to_float(ob), acc);
    }
    return fmaf(chunk_dot4(wq, xp), half_bits_to_float(sb), acc);
  }

  // acc[b][t] = this lane's share of row_b . act_t (same activations for every batch)
  template <int TT>
  __device__ __forceinline__ void dot_shared(const RowGeom& g, const _Float16* act, int stride, int T,
                                             float acc[NB][TT], const float* xs = nullptr, int xs_stride = 0) const {
    const int lane = threadIdx.x & 63;
    constexpr int EPC = BITS == 4 ? 32 : 16;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[b][t] = 0.f;
#pragma unroll
    for (int m = 0; m < MAXCPL; ++m) {
      if (m < g.cpl) {
        const int c = (lane % g.lpr) + g.lpr * m;
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          if (t < T) {
            const _Float16* a = act + (size_t)t * stride + EPC * c;
            if (BITS == 4) {
              h2 xp[16];
              act32(a, xp);
              const float xsum = AFF ? xs[(size_t)t * xs_stride + c] : 0.f;
#pragma unroll
              for (int b = 0; b < NB; ++b) acc[b][t] = chunk4(q[b][m], xp, s[b][m], o[b][m], xsum, acc[b][t]);
            } else {
              h2 xp[8];
              act16(a, xp);
#pragma unroll
              for (int b = 0; b < NB; ++b) acc[b][t] = fmaf(chunk_dot8(q[b][m], xp), half_bits_to_float(s[b][m]), acc[b][t]);
            }
          }
        }
      }
    }
  }

  // acc[b] = this lane's share of row_b . act_b (one activation vector per batch;
  // AFF: xs[b] its chunk sums)
  __device__ __forceinline__ void dot_per_batch(const RowGeom& g, const _Float16* const act[NB], float acc[NB],
                                                const float* const* xs = nullptr) const {
    const int lane = threadIdx.x & 63;
    constexpr int EPC = BITS == 4 ? 32 : 16;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      acc[b] = 0.f;
      if (act[b] == nullptr) continue;
#pragma unroll
      for (int m = 0; m < MAXCPL; ++m) {
        if (m < g.cpl) {
          const int c = (lane % g.lpr) + g.lpr * m;
          if (BITS == 4) {
            h2 xp[16];
            act32(act[b] + EPC * c, xp);
            acc[b] = chunk4(q[b][m], xp, s[b][m], o[b][m], AFF ? xs[b][c] : 0.f, acc[b]);
          } else {
            h2 xp[8];
            act16(act[b] + EPC * c, xp);
            acc[b] = fmaf(chunk_dot8(q[b][m], xp), half_bits_to_float(s[b][m]), acc[b]);
          }
        }
      }
    }
  }
};

}  // namespace moe
