// Multi-token path of the routed MoE block: grouped GEMMs on MFMA.
//
// The same block as the few-token path (the Chimera notebook, section 5; the
// router ordering of section 5.2; int8 group-64 router rows stacked with the
// shared gate, the TensorFold PR "Design"), organised for many tokens:
//   1. router GEMM          logits[T][E+1]   (int8 rows, MFMA, per-group scales; for
//                           the complete block at few tokens in two K halves, added
//                           by the top-k; above 2048 tokens one workgroup per 32
//                           tokens over every block of router rows)
//   2. top-k per token      ids, renormalised weights, sigma
//   3. bucketing            (token, slot) pairs grouped by expert; tiles of up
//                           to 128 rows per expert, shared tiles (2 and 3 run
//                           in one launch for the complete block: the last
//                           top-k workgroup sorts; above 1024 tokens the sort
//                           is spread over the grid in three launches)
//   4. gate/up GEMM         h[row][I] = silu(x W_gate^T) * (x W_up^T)   (fp16)
//   5. down GEMM            y[t*k+i][H] = w * (h W_down^T)                (fp16)
//   6. combine              out[t] = sum_i y[t*k+i] + sigma_t * s[t]
// Each tile streams its expert's weights once; a tile's rows are the tokens
// routed to that expert.  For the sub-block of a decoder layer (the same
// notebook, sections 7 and 10) the router GEMM also applies the post-attention
// RMSNorm and writes the normalised rows the expert GEMMs read, and the combine
// adds the residual.
#include "chunk.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// MFMA 32x32x16 f16 operand layout used throughout: lane l works on row
// (l % 32) of a 32-row operand and on K offsets 32*(l/32) + 8*s .. +8 of each
// 64-wide group in MFMA step s (0..3).  A and B use the same K assignment, so
// the products pair up; the 16 K values of one step lie in one group.
// Accumulator element i of lane l is row 8*(i/4) + 4*(l/32) + (i%4), column
// l % 32.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int acc_row(int i) { return 8 * (i >> 2) + 4 * ((threadIdx.x & 63) >> 5) + (i & 3); }

__device__ __forceinline__ h8 pack8(const h2 w[4]) {
  h8 r;
  r[0] = w[0][0]; r[1] = w[0][1]; r[2] = w[1][0]; r[3] = w[1][1];
  r[4] = w[2][0]; r[5] = w[2][1]; r[6] = w[3][0]; r[7] = w[3][1];
  return r;
}

// 8 activations (one 16-byte chunk, natural order) -> MFMA operand in the
// (0,4,1,5,2,6,3,7) order of the weight conversion
__device__ __forceinline__ h8 act_operand(uint4 v) {
  const uint32_t x[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
  perm8_words(x, o);
  return __builtin_bit_cast(h8, make_uint4(o[0], o[1], o[2], o[3]));
}

// ---------------------------------------------------------------------------
// Range-checked buffer loads.  A masked row, column or group gets an offset
// outside its resource and reads zeros, so loads are issued unconditionally
// and no load feeds a select (a load under a branch, or one whose value is
// selected at once, makes the compiler wait for it where it is issued).
// ---------------------------------------------------------------------------
static constexpr uint32_t kOob = 0x80000000u;  // an offset outside every resource: reads return zero

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// the same for a buffer-load result
__device__ __forceinline__ h8 act_operand(u32x4 v) {
  const uint32_t x[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
  perm8_words(x, o);
  return __builtin_bit_cast(h8, make_uint4(o[0], o[1], o[2], o[3]));
}

// raw (stride 0) resource; the config word selects 32-bit data format (gfx9).
// Base and size must be workgroup-uniform: they are moved to scalar registers
// here, so the compiler never wraps a load in a per-lane resource loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b), hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// ---------------------------------------------------------------------------
// 1. router GEMM: 32 tokens x 32 rows per workgroup; the kRouterWaves waves
//    take interleaved 64-groups of K and are summed through LDS.  At hidden
//    2048 each wave's four groups are one batch of loads, so the kernel waits
//    on memory once.  The loads are coalesced (consecutive lanes read
//    consecutive 16-byte pieces of one row) and go through the wave's own LDS
//    slice into the MFMA operand layout, where each lane works on its own row:
//    loads in that layout make the texture addresser take the lanes one at a
//    time.  The scales are applied per group to fp32 partial sums, so routing
//    sees logits accurate to fp32 rounding.
// ---------------------------------------------------------------------------
static constexpr int kRouterWaves = 8;
static constexpr int kRxStride = 9;  // 16-byte chunks per LDS row of activations (8 + 1 against bank conflicts)
static constexpr int kRwStride = 5;  // ... of router codes (4 + 1)

// With gridDim.z = 2 (the complete block, few tokens) workgroup z takes K groups
// [z ngr / 2, (z + 1) ngr / 2) and writes its partial sums to logits (z = 0)
// or logits_hi (z = 1); the top-k adds the two in that order.  The staging
// slices and the partial-sum buffer share their LDS (a barrier separates
// them), so two workgroups fit on a compute unit.
static constexpr int kRouterStage = kRouterWaves * 32 * (kRxStride + kRwStride);  // uint4s
static constexpr int kRouterRed = kRouterWaves * 16 * 64 / 4;                        // uint4s
// BATCH: K groups per wave in flight at once (2 for the K halves, whose
// registers then let two workgroups share a compute unit)
template <int BATCH>
__global__ __launch_bounds__(64 * kRouterWaves, BATCH == 2 ? 4 : 1) void router_gemm_kernel(ChunkArgs a) {
  __shared__ uint4 router_lds[kRouterStage > kRouterRed ? kRouterStage : kRouterRed];
  auto red = reinterpret_cast<float (*)[16][64]>(router_lds);
  auto stage = reinterpret_cast<uint4 (*)[32 * (kRxStride + kRwStride)]>(router_lds);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gb = blockIdx.z * (a.H / kGroup) / gridDim.z, ge = (blockIdx.z + 1) * (a.H / kGroup) / gridDim.z;
  const int m = lane & 31, g = lane >> 5;
  const int t0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int r = r0 + m;  // B row (router row) of this MFMA lane
  const int nrows = a.E + 1, H = a.H, ngr = H / kGroup;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)a.T * H * 2u);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.router_q, (uint32_t)nrows * H);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.router_s, (uint32_t)nrows * ngr * 2u);
  // coalesced pieces: activations 32 rows x 8 chunks of a group (4 per lane),
  // codes 32 rows x 4 chunks (2 per lane)
  uint32_t xoff[4], qoff[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int idx = 64 * j + lane, row = idx >> 3;
    xoff[j] = t0 + row < a.T ? (uint32_t)(t0 + row) * H * 2u + 16u * (idx & 7) : kOob;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int idx = 64 * j + lane, row = idx >> 2;
    qoff[j] = r0 + row < nrows ? (uint32_t)(r0 + row) * H + 16u * (idx & 3) : kOob;
  }
  const uint32_t soff = r < nrows ? (uint32_t)r * ngr * 2u : kOob;
  // The sub-block (the Chimera notebook, sections 7 and 10: post-attention
  // RMSNorm in front of the block): a first pass sums each token's squares
  // (fixed order, so every row block derives the same binary16 activations);
  // the GEMM then scales each activation piece by its token's reciprocal RMS
  // and the gain, and the first row block writes them out for the expert GEMMs.
  __shared__ float s_rn[32];
  const bool sub = a.gain != nullptr;  // uniform
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.gain, sub ? (uint32_t)H * 2u : 0u);
  const bool one_batch = ngr <= kRouterWaves * BATCH;  // H <= 2048: the batch holds the wave's whole share
  // reciprocal RMS of the 32 tokens from each lane's partial sums of squares
  // of rows 8j + lane / 8 (four rows per lane)
  auto finish_rn = [&](float ss[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // the 8 lanes of one row (lanes 8m .. 8m + 7)
      ss[j] += __shfl_xor(ss[j], 1, 64);
      ss[j] += __shfl_xor(ss[j], 2, 64);
      ss[j] += __shfl_xor(ss[j], 4, 64);
      if ((lane & 7) == 0) red[wave][j][lane >> 3] = ss[j];
    }
    __syncthreads();
    if (threadIdx.x < 32) {
      const int row = threadIdx.x;
      float t = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kRouterWaves; ++w2) t += red[w2][row >> 3][row & 7];
      s_rn[row] = 1.0f / sqrtf(t / (float)H + a.eps);
    }
    __syncthreads();
  };
  auto add_squares = [&](float ss[4], const u32x4 v[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const h8 hv = __builtin_bit_cast(h8, v[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss[j] = fmaf((float)hv[i], (float)hv[i], ss[j]);
    }
  };
  if (sub && !one_batch) {  // wider rows: a first pass over x for the sums of squares
    float ss[4] = {0.f, 0.f, 0.f, 0.f};
    for (int g0 = wave; g0 < ngr; g0 += kRouterWaves * BATCH) {
      u32x4 v[BATCH][4];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int gi = g0 + kRouterWaves * u;
        const uint32_t kx = gi < ngr ? 128u * gi : kOob;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[u][j] = __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[j] + kx, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) add_squares(ss, v[u]);
    }
    finish_rn(ss);
  }
  const __amdgpu_buffer_rsrc_t rxn = make_rsrc(a.xn, sub && blockIdx.y == 0 ? (uint32_t)a.T * H * 2u : 0u);
  uint4* xs = stage[wave];
  uint4* wsl = stage[wave] + 32 * kRxStride;
  f16v acc = {};
  // Every wave runs the body at least once, also a wave with no group in
  // [gb, ge) (narrow rows, or a K half): its loads are all out of range and
  // read zeros, and it joins the workgroup barriers of the norm below.
  for (int g0 = gb + wave;; g0 += kRouterWaves * BATCH) {
    u32x4 xa[BATCH][4], wb[BATCH][2], gn[BATCH];
    uint16_t sc[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int gi = g0 + kRouterWaves * u;
      const bool ok = gi < ge;  // uniform
      const uint32_t kx = ok ? 128u * gi : kOob, kq = ok ? 64u * gi : kOob, ks = ok ? 2u * gi : kOob;
#pragma unroll
      for (int j = 0; j < 4; ++j) xa[u][j] = __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[j] + kx, 0, 0);
#pragma unroll
      for (int j = 0; j < 2; ++j) wb[u][j] = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff[j] + kq, 0, 0);
      sc[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff + ks, 0, 0);
      gn[u] = __builtin_amdgcn_raw_buffer_load_b128(rg, ok ? 128u * gi + 16u * (lane & 7) : kOob, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);  // the whole batch in flight before any use
    if (sub && one_batch) {  // the batch holds the wave's share of every row
      float ss[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < BATCH; ++u) add_squares(ss, xa[u]);
      finish_rn(ss);
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (sub) {  // binary16(x * rsqrt(mean x^2 + eps) * gain), kept for the expert GEMMs
        const h8 gv = __builtin_bit_cast(h8, gn[u]);
        const int gi = g0 + kRouterWaves * u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float rn = s_rn[(64 * j + lane) >> 3];
          h8 hv = __builtin_bit_cast(h8, xa[u][j]);
#pragma unroll
          for (int i = 0; i < 8; ++i) hv[i] = (_Float16)((float)hv[i] * rn * ((float)gv[i] + a.gain_add));
          xa[u][j] = __builtin_bit_cast(u32x4, hv);
          if (gi < ge) __builtin_amdgcn_raw_buffer_store_b128(xa[u][j], rxn, xoff[j] + 128u * gi, 0, 0);
        }
      }
      // the wave's slice: written by all its lanes, then read in MFMA layout
      // (LDS operations of one wave complete in order)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = 64 * j + lane;
        xs[(idx >> 3) * kRxStride + (idx & 7)] = __builtin_bit_cast(uint4, act_operand(xa[u][j]));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int idx = 64 * j + lane;
        wsl[(idx >> 2) * kRwStride + (idx & 3)] = __builtin_bit_cast(uint4, wb[u][j]);
      }
      __builtin_amdgcn_wave_barrier();
      f16v p = {};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const h8 av = __builtin_bit_cast(h8, xs[m * kRxStride + 4 * g + st]);
        const uint2 wq = reinterpret_cast<const uint2*>(wsl + m * kRwStride + 2 * g + (st >> 1))[st & 1];
        h2 w[4];
        int8x8_to_h2x4(wq.x, wq.y, w);
        p = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pack8(w), p, 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();
      const float scf = half_bits_to_float(sc[u]);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = fmaf(p[i], scf, acc[i]);
    }
    if (g0 + kRouterWaves * BATCH >= ge) break;
  }
  __syncthreads();  // every wave is done with its staging slice (red shares the LDS)
#pragma unroll
  for (int i = 0; i < 16; ++i) red[wave][i][lane] = acc[i];
  __syncthreads();
  // the 8 waves' partial sums, added in wave order; wave w writes accumulator
  // elements i = w, w + 8 (the lanes' rows and columns as in the MFMA layout)
  float* const lo = blockIdx.z ? a.logits_hi : a.logits;
  if (r < nrows) {
#pragma unroll
    for (int i = wave; i < 16; i += kRouterWaves) {
      const int tt = t0 + acc_row(i);
      float v = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kRouterWaves; ++w2) v += red[w2][i][lane];
      if (tt < a.T) lo[(size_t)tt * nrows + r] = v;
    }
  }
}

// Many tokens (T > kRouterRowsT, hidden <= 2048, whole K): one workgroup per
// 32 tokens runs every block of 32 router rows.  Its activations are loaded
// once (in the sub-block also normalised and written out once) and kept in
// registers in the MFMA operand layout; each row block's codes and scales are
// loaded while the previous block is multiplied.  The one-block-per-workgroup
// form above reloads the tokens' activations for every row block and runs
// nine times as many short workgroups, which at many tokens queue in rounds.
static constexpr int kRouterRowsT = 2048;
static_assert(kRouterWaves * 16 * 64 * sizeof(float) <= kRouterWaves * 32 * kRxStride * sizeof(uint4),
              "the partial sums fit in the activation staging slices");

__global__ __launch_bounds__(64 * kRouterWaves, 1) void router_rows_kernel(ChunkArgs a) {
  __shared__ uint4 lds_x[kRouterWaves][32 * kRxStride];  // activation staging, then the partial sums
  __shared__ uint4 lds_w[kRouterWaves][32 * kRwStride];
  __shared__ float s_rn[32];
  auto red = reinterpret_cast<float (*)[16][64]>(&lds_x[0][0]);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = lane & 31, g = lane >> 5;
  const int t0 = blockIdx.x * 32;
  const int nrows = a.E + 1, H = a.H, ngr = H / kGroup;  // ngr <= 4 * kRouterWaves
  const int nrb = (nrows + 31) / 32;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)a.T * H * 2u);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.router_q, (uint32_t)nrows * H);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.router_s, (uint32_t)nrows * ngr * 2u);
  const bool sub = a.gain != nullptr;  // uniform
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.gain, sub ? (uint32_t)H * 2u : 0u);
  const __amdgpu_buffer_rsrc_t rxn = make_rsrc(a.xn, sub ? (uint32_t)a.T * H * 2u : 0u);
  uint32_t xoff[4];  // coalesced pieces: 32 rows x 8 chunks of a group, 4 per lane
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int idx = 64 * j + lane, row = idx >> 3;
    xoff[j] = t0 + row < a.T ? (uint32_t)(t0 + row) * H * 2u + 16u * (idx & 7) : kOob;
  }
  // the wave's groups: gi = wave + kRouterWaves * u
  u32x4 xa[4][4], gn[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int gi = wave + kRouterWaves * u;
    const uint32_t kx = gi < ngr ? 128u * gi : kOob;
#pragma unroll
    for (int j = 0; j < 4; ++j) xa[u][j] = __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[j] + kx, 0, 0);
    gn[u] = __builtin_amdgcn_raw_buffer_load_b128(rg, gi < ngr ? 128u * gi + 16u * (lane & 7) : kOob, 0, 0);
  }
  // codes (32 rows x 4 chunks of a group, 2 per lane) and scales of row block rb
  auto load_codes = [&](int rb, u32x4 (&w)[4][2], uint16_t (&sc)[4]) {
    const int r0 = rb * 32;
    uint32_t qoff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int idx = 64 * j + lane, row = idx >> 2;
      qoff[j] = r0 + row < nrows ? (uint32_t)(r0 + row) * H + 16u * (idx & 3) : kOob;
    }
    const uint32_t soff = r0 + m < nrows ? (uint32_t)(r0 + m) * ngr * 2u : kOob;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int gi = wave + kRouterWaves * u;
      const bool ok = gi < ngr;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        w[u][j] = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff[j] + (ok ? 64u * gi : kOob), 0, 0);
      sc[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff + (ok ? 2u * gi : kOob), 0, 0);
    }
  };
  u32x4 wb[4][2];
  uint16_t sc[4];
  load_codes(0, wb, sc);
  __builtin_amdgcn_sched_barrier(0);  // activations and the first codes in flight before any use
  if (sub) {  // reciprocal RMS of the 32 tokens (rows 8j + lane / 8 of this lane's pieces)
    float ss[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const h8 hv = __builtin_bit_cast(h8, xa[u][j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) ss[j] = fmaf((float)hv[i], (float)hv[i], ss[j]);
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // the 8 lanes of one row
      ss[j] += __shfl_xor(ss[j], 1, 64);
      ss[j] += __shfl_xor(ss[j], 2, 64);
      ss[j] += __shfl_xor(ss[j], 4, 64);
      if ((lane & 7) == 0) red[wave][j][lane >> 3] = ss[j];
    }
    __syncthreads();
    if (threadIdx.x < 32) {
      const int row = threadIdx.x;
      float t = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kRouterWaves; ++w2) t += red[w2][row >> 3][row & 7];
      s_rn[row] = 1.0f / sqrtf(t / (float)H + a.eps);
    }
    __syncthreads();
  }
  // the activations into registers in the MFMA layout, through the wave's slice
  // (LDS operations of one wave complete in order)
  uint4* const xs = lds_x[wave];
  h8 av[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int gi = wave + kRouterWaves * u;
    if (sub) {  // binary16(x * rsqrt(mean x^2 + eps) * gain), kept for the expert GEMMs
      const h8 gv = __builtin_bit_cast(h8, gn[u]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float rn = s_rn[(64 * j + lane) >> 3];
        h8 hv = __builtin_bit_cast(h8, xa[u][j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = (_Float16)((float)hv[i] * rn * ((float)gv[i] + a.gain_add));
        xa[u][j] = __builtin_bit_cast(u32x4, hv);
        if (gi < ngr) __builtin_amdgcn_raw_buffer_store_b128(xa[u][j], rxn, xoff[j] + 128u * gi, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = 64 * j + lane;
      xs[(idx >> 3) * kRxStride + (idx & 7)] = __builtin_bit_cast(uint4, act_operand(xa[u][j]));
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int st = 0; st < 4; ++st) av[u][st] = __builtin_bit_cast(h8, xs[m * kRxStride + 4 * g + st]);
    __builtin_amdgcn_wave_barrier();
  }
  uint4* const wsl = lds_w[wave];
  for (int rb = 0; rb < nrb; ++rb) {
    u32x4 wn[4][2];
    uint16_t scn[4];
    load_codes(min(rb + 1, nrb - 1), wn, scn);  // the next block's (the last block's again at the end)
    f16v acc = {};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int idx = 64 * j + lane;
        wsl[(idx >> 2) * kRwStride + (idx & 3)] = __builtin_bit_cast(uint4, wb[u][j]);
      }
      __builtin_amdgcn_wave_barrier();
      f16v p = {};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const uint2 wq = reinterpret_cast<const uint2*>(wsl + m * kRwStride + 2 * g + (st >> 1))[st & 1];
        h2 w[4];
        int8x8_to_h2x4(wq.x, wq.y, w);
        p = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[u][st], pack8(w), p, 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();
      const float scf = half_bits_to_float(sc[u]);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = fmaf(p[i], scf, acc[i]);
    }
    __syncthreads();  // every wave is past its staging reads and the previous block's sums
#pragma unroll
    for (int i = 0; i < 16; ++i) red[wave][i][lane] = acc[i];
    __syncthreads();
    const int r = rb * 32 + m;  // router row of this lane's column
    if (r < nrows) {
#pragma unroll
      for (int i = wave; i < 16; i += kRouterWaves) {  // the 8 waves' sums in wave order
        const int tt = t0 + acc_row(i);
        float v = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kRouterWaves; ++w2) v += red[w2][i][lane];
        if (tt < a.T) a.logits[(size_t)tt * nrows + r] = v;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      wb[u][0] = wn[u][0];
      wb[u][1] = wn[u][1];
      sc[u] = scn[u];
    }
  }
}

// ---------------------------------------------------------------------------
// 2. top-k: one wave per token
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void topk_kernel(ChunkArgs a) {
  __shared__ TopkScratch sc[4];
  __shared__ int ids[4][kMaxTopK];
  __shared__ float w[4][kMaxTopK];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.T) return;  // whole waves: no workgroup barrier below
  const int nrows = a.E + 1;
  const float* lg = a.logits + (size_t)t * nrows;
  // all loads issued before any use (clamped indices: entries past E are
  // ignored by the ranking)
  float gate = lg[a.E];
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = lg[min(4 * lane + j, a.E)];
  if (a.logits_hi) {  // the second K half's partial sums, added after the first
    const float* lh = a.logits_hi + (size_t)t * nrows;
    gate += lh[a.E];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] += lh[min(4 * lane + j, a.E)];
  }
  wave_topk(v, a.E, a.k, ids[wave], w[wave], sc[wave]);
  __builtin_amdgcn_wave_barrier();
  if (lane < a.k) {
    a.ids[(size_t)t * a.k + lane] = ids[wave][lane];
    a.wts[(size_t)t * a.k + lane] = w[wave][lane];
  }
  if (lane == 0) a.sigma[t] = sigmoid_f(gate);
}

// ---------------------------------------------------------------------------
// 3. bucketing: one workgroup of 1024 threads (16 waves)
//
// Pairs p = t*k + i are grouped by expert: a counting sort.  Each wave owns
// a contiguous run of pairs and its own per-expert counters in LDS, and
// places inside the wave's share of an expert's run come from LDS atomic adds
// on those counters.  Only one wave touches a counter, and the lanes of one
// instruction are served in a fixed order, so the order is the same in every
// call on the same routing.  That matters: it decides which pairs fall into
// an expert's last tile, which may take another MFMA shape (and rounding)
// than its full tiles.  Each expert's rows are cut into kTileRows-row tiles
// and one last tile of 1..kTileRows rows, which uses only as many 32-row MFMA
// blocks as it needs (or the narrow path, for at most kNarrowRows rows).
// ---------------------------------------------------------------------------
// the tile's MFMA row blocks of 32; 0 marks a narrow tile (at most kNarrowRows rows)
__device__ __forceinline__ int4 make_tile(int e, int r0, int rows) {
  return make_int4(e, r0, rows, rows <= kNarrowRows ? 0 : (rows + 31) / 32);
}

// shared-expert tile st: tokens st * kSharedRows .. (expert -1; never narrow)
__device__ __forceinline__ int4 shared_tile(int st, int T) {
  const int r0 = st * kSharedRows, rows = min(kSharedRows, T - r0);
  return make_int4(-1, r0, rows, (rows + 31) / 32);
}

static constexpr int kTileClasses = kTileRows / 32 + 1;  // cost classes: 32-row blocks, 0 = narrow

// Slot of the j-th tile of the heaviest class (n tiles, slots 0..n-1).  The
// GEMM kernels run tile s on XCD s % 8, so the class is filled column by
// column of an 8-wide grid: consecutive j, which are one expert's tiles, share
// an XCD, and its L2 fetches the expert's weights once for all of them.
struct TopSlots {
  int R;   // rows of the grid
  int fc;  // columns with R rows (the others have R - 1)
  __device__ __forceinline__ explicit TopSlots(int n) : R((n + 7) / 8), fc(n - 8 * ((n + 7) / 8 - 1)) {}
  // column c and row rho of the j-th tile
  __device__ __forceinline__ void at(int j, int& c, int& rho) const {
    if (j < fc * R) {
      c = j / R;
      rho = j - c * R;
    } else {
      const int jj = j - fc * R;
      c = fc + jj / (R - 1);
      rho = jj - (c - fc) * (R - 1);
    }
  }
  // the (j+1)-th tile from the j-th: down the column, then to the next one
  __device__ __forceinline__ void next(int& c, int& rho) const {
    if (++rho == (c < fc ? R : R - 1)) {
      rho = 0;
      ++c;
    }
  }
};
__device__ __forceinline__ int top_slot(int j, int n) {
  int c, rho;
  TopSlots(n).at(j, c, rho);
  return 8 * rho + c;
}

// ids and routing weights of pairs: ordinary loads, or device-coherent loads
// when other workgroups of the same launch wrote them
template <bool CO>
__device__ __forceinline__ int load_id(const int32_t* p) {
  if (CO) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}
template <bool CO>
__device__ __forceinline__ float load_wt(const float* p) {
  if (CO)
    return __builtin_bit_cast(float, __hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT));
  return *p;
}

// LDS of the bucketing.  bucket_clear must run, and a workgroup barrier
// follow it, before bucket_body.
struct BucketLds {
  int cnt[16][kMaxExperts];      // pairs per wave and expert, then the wave's next place
  int off[kMaxExperts];          // first place of each expert's run
  int cls[2][kTileClasses];      // tiles per cost class, then each class's next slot
  int total;                     // pairs kept (ids in [0, E))
};

__device__ __forceinline__ void bucket_clear(BucketLds& s) {
  for (int i = threadIdx.x; i < 16 * kMaxExperts; i += blockDim.x) (&s.cnt[0][0])[i] = 0;
  if (threadIdx.x < kTileClasses) s.cls[0][threadIdx.x] = 0;
}

// The tile list from the experts' pair counts: count_of(e) is called once
// by thread e < kMaxExperts (0 for e >= E).  On return s.off holds each
// expert's first place, the tiles and the tile count are written, and every
// thread has passed the barrier after the scan.  Needs kMaxExperts threads.
template <class CountOf>
__device__ __forceinline__ void bucket_tiles(const ChunkArgs& a, BucketLds& s, CountOf count_of) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int E = a.E;
  constexpr int top = kTileRows / 32;  // the heaviest class
  if (threadIdx.x < kMaxExperts) {  // each expert's count; tiles per cost class
    const int e = threadIdx.x;
    const int tot = count_of(e);
    s.off[e] = tot;  // the count for now
    if (tot >= kTileRows) atomicAdd(&s.cls[0][top], tot / kTileRows);
    const int tc = tot % kTileRows ? make_tile(e, 0, tot % kTileRows).w : -1;
#pragma unroll
    for (int c = 0; c < kTileClasses; ++c) {
      const uint64_t m = __ballot(tc == c);
      if (m && lane == 0) atomicAdd(&s.cls[0][c], __popcll(m));
    }
  }
  if (threadIdx.x == blockDim.x - 1 && a.shared_tiles > 0) {  // all full but perhaps the last
    const int ns = a.shared_tiles;
    if (ns > 1) atomicAdd(&s.cls[0][shared_tile(0, a.T).w], ns - 1);
    atomicAdd(&s.cls[0][shared_tile(ns - 1, a.T).w], 1);
  }
  __syncthreads();
  if (wave == 0) {  // exclusive scan of counts (E <= 256: 4 per lane)
    int c[4];
    int sc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      c[j] = e < E ? s.off[e] : 0;
      sc += c[j];
    }
    int ic = sc;
    for (int d = 1; d < 64; d <<= 1) {
      const int uc = __shfl_up(ic, d, 64);
      if (lane >= d) ic += uc;
    }
    int ec = ic - sc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s.off[4 * lane + j] = ec;
      ec += c[j];
    }
    if (lane == 63) s.total = ic;
    if (lane == 0) {  // classes in decreasing cost: the tile list starts with the heaviest tiles
      int base = 0;
      for (int c2 = kTileClasses - 1; c2 >= 0; --c2) {
        s.cls[1][c2] = base;
        base += s.cls[0][c2];
      }
      *a.n_tiles = base;
    }
  }
  __syncthreads();
  {
    // Tiles in cost order (the order inside a class is immaterial: every
    // output row and column belongs to exactly one tile).  An expert's tiles
    // of the heaviest class take one run of slots.
    const int total = s.total;
    const int n_top = s.cls[0][top];
    if (threadIdx.x < kMaxExperts) {
      const int e = threadIdx.x;
      const int start = e < E ? s.off[e] : 0;
      const int end = e + 1 < E ? s.off[e + 1] : (e < E ? total : 0);
      const int tail = (end - start) % kTileRows;
      const int tc = tail ? make_tile(e, 0, tail).w : -1;
      const int run = (end - start) / kTileRows + (tc == top ? 1 : 0);  // the expert's tiles of the heaviest class
      int r = start;
      if (run) {  // one division for the run's first slot, then a walk down the grid
        const TopSlots ts(n_top);
        int c, rho;
        ts.at(atomicAdd(&s.cls[1][top], run), c, rho);
        for (int i = 0; i < run; ++i, r += kTileRows) {
          a.tiles[8 * rho + c] = make_tile(e, r, min(kTileRows, end - r));
          ts.next(c, rho);
        }
      }
      if (tc >= 0 && tc != top) a.tiles[atomicAdd(&s.cls[1][tc], 1)] = make_tile(e, r, end - r);  // a lighter last tile
    }
    for (int st = threadIdx.x; st < a.shared_tiles; st += blockDim.x) {
      const int4 t = shared_tile(st, a.T);
      const int ti = atomicAdd(&s.cls[1][t.w], 1);
      a.tiles[t.w == top ? top_slot(ti, n_top) : ti] = t;  // the heaviest class's slots follow top_slot
    }
  }
}

template <bool CO>
__device__ __forceinline__ void bucket_body(const ChunkArgs& a, BucketLds& s) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int P = a.T * a.k;
  const int E = a.E;
  const int per = (P + 15) / 16;
  const int p_begin = min(P, wave * per), p_end = min(P, p_begin + per);

  // counts (ids outside [0, E) are dropped: they never index weights).  Ids
  // are loaded kBatch rounds at a time with clamped (always valid) indices,
  // so the loads are in flight together.  The first batch of ids and routing
  // weights stays in registers for the scatter below (with T * k <= 16 * 64 *
  // kBatch it is the wave's whole share).
  constexpr int kBatch = 4;
  int ev0[kBatch];
  float wv0[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    ev0[u] = load_id<CO>(a.ids + min(p_begin + 64 * u + lane, P - 1));
    wv0[u] = load_wt<CO>(a.wts + min(p_begin + 64 * u + lane, P - 1));
  }
  auto count = [&](int p0, const int* ev) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = p0 + 64 * u + lane;
      const int e = p < p_end ? ev[u] : -1;
      if (e >= 0 && e < E) atomicAdd(&s.cnt[wave][e], 1);
    }
  };
  count(p_begin, ev0);
  for (int p0 = p_begin + 64 * kBatch; p0 < p_end; p0 += 64 * kBatch) {
    int ev[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) ev[u] = load_id<CO>(a.ids + min(p0 + 64 * u + lane, P - 1));
    count(p0, ev);
  }
  __syncthreads();
  bucket_tiles(a, s, [&](int e) {  // the waves' counts -> their first places in the expert's run
    int tot = 0;
    if (e < E)
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        const int c = s.cnt[w][e];
        s.cnt[w][e] = tot;
        tot += c;
      }
    return tot;
  });
  // scatter: each pair's place in its expert's run, with its routing weight
  // (so the down GEMM reads both by place)
  auto scatter = [&](int p0, const int* ev, const float* wv) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = p0 + 64 * u + lane;
      const int e = p < p_end ? ev[u] : -1;
      if (e >= 0 && e < E) {
        const int pos = s.off[e] + atomicAdd(&s.cnt[wave][e], 1);
        a.sorted_pair[pos] = p;
        a.sorted_wt[pos] = wv[u];
      }
    }
  };
  scatter(p_begin, ev0, wv0);
  for (int p0 = p_begin + 64 * kBatch; p0 < p_end; p0 += 64 * kBatch) {
    int ev[kBatch];
    float wv[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      ev[u] = load_id<CO>(a.ids + min(p0 + 64 * u + lane, P - 1));
      wv[u] = load_wt<CO>(a.wts + min(p0 + 64 * u + lane, P - 1));
    }
    scatter(p0, ev, wv);
  }
}

// caller-supplied routing (the routed half alone)
__global__ __launch_bounds__(1024) void bucket_kernel(ChunkArgs a) {
  __shared__ BucketLds bs;
  bucket_clear(bs);
  __syncthreads();
  bucket_body<false>(a, bs);
}

// ---------------------------------------------------------------------------
// 2 + 3 in one launch (the complete block): each wave ranks one token as in
// topk_kernel (four to sixteen tokens per workgroup, so that the ranking is
// spread over many compute units), and the last workgroup to finish, found
// with a device-scope counter, sorts the pairs.  ids and weights are written with device-coherent
// stores and acknowledged before the counter moves, and that workgroup reads
// them back with device-coherent loads, so no L2 serves it a stale copy.  No
// workgroup waits for another: the kernel always drains.
// ---------------------------------------------------------------------------
static constexpr int kTopkBucketWaves = 16;

// Token t's logits ranked by the calling wave (ids and weights in rank
// order into its LDS rows); returns the shared-gate logit.
__device__ __forceinline__ float rank_token(const ChunkArgs& a, int t, int* ids, float* w, TopkScratch& sc) {
  const int lane = threadIdx.x & 63;
  const int nrows = a.E + 1;
  const float* lg = a.logits + (size_t)t * nrows;
  float gate = lg[a.E];
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = lg[min(4 * lane + j, a.E)];
  if (a.logits_hi) {  // the second K half's partial sums, added after the first
    const float* lh = a.logits_hi + (size_t)t * nrows;
    gate += lh[a.E];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] += lh[min(4 * lane + j, a.E)];
  }
  wave_topk(v, a.E, a.k, ids, w, sc);
  __builtin_amdgcn_wave_barrier();
  return gate;
}

__global__ __launch_bounds__(64 * kTopkBucketWaves) void topk_bucket_kernel(ChunkArgs a) {
  __shared__ TopkScratch sc[kTopkBucketWaves];
  __shared__ int ids[kTopkBucketWaves][kMaxTopK];
  __shared__ float w[kTopkBucketWaves][kMaxTopK];
  __shared__ BucketLds bs;
  __shared__ int s_last;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tpw = (a.T + gridDim.x - 1) / gridDim.x;  // tokens per workgroup (at most kTopkBucketWaves)
  const int t = blockIdx.x * tpw + wave;
  if (wave < tpw && t < a.T) {
    const float gate = rank_token(a, t, ids[wave], w[wave], sc[wave]);
    if (lane < a.k) {
      __hip_atomic_store(a.ids + (size_t)t * a.k + lane, ids[wave][lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(reinterpret_cast<uint32_t*>(a.wts) + (size_t)t * a.k + lane,
                         __builtin_bit_cast(uint32_t, w[wave][lane]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane == 0) a.sigma[t] = sigmoid_f(gate);
  }
  bucket_clear(bs);  // while the stores drain (only the last workgroup uses it)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are acknowledged
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(a.route_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x == 0) __hip_atomic_store(a.route_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  bucket_body<true>(a, bs);
}

// ---------------------------------------------------------------------------
// 2 + 3 for many tokens (T > kGridBucketT).  One workgroup sorting every pair
// is bound by its compute unit's scattered stores (933 us at 65536 tokens),
// so the sort is spread over the grid in three launches:
//   topk_count_kernel      each workgroup ranks kTopkBucketWaves tokens and
//                          writes its per-expert counts into column e of
//                          wg_cnt ([E][workgroups])
//   bucket_scan_kernel     one workgroup per expert turns its row into
//                          exclusive bases over the workgroups; the last one
//                          to finish lays out the tile list
//   bucket_scatter_kernel  one wave per top-k workgroup's pairs: place =
//                          expert offset + that workgroup's base + the
//                          wave's LDS rank
// Inside an expert's run the pairs come in workgroup order, then in the order
// one wave's LDS atomics hand out, the same in every call on the same routing.
// ---------------------------------------------------------------------------
static constexpr int kGridBucketT = 1024;

__global__ __launch_bounds__(64 * kTopkBucketWaves) void topk_count_kernel(ChunkArgs a) {
  __shared__ TopkScratch sc[kTopkBucketWaves];
  __shared__ int ids[kTopkBucketWaves][kMaxTopK];
  __shared__ float w[kTopkBucketWaves][kMaxTopK];
  __shared__ int hist[kMaxExperts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkBucketWaves + wave;
  for (int i = threadIdx.x; i < kMaxExperts; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  if (t < a.T) {
    const float gate = rank_token(a, t, ids[wave], w[wave], sc[wave]);
    if (lane < a.k) {
      a.ids[(size_t)t * a.k + lane] = ids[wave][lane];
      a.wts[(size_t)t * a.k + lane] = w[wave][lane];
      atomicAdd(&hist[ids[wave][lane]], 1);
    }
    if (lane == 0) a.sigma[t] = sigmoid_f(gate);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) a.wg_cnt[(size_t)e * gridDim.x + blockIdx.x] = hist[e];
}

__global__ __launch_bounds__(256) void bucket_scan_kernel(ChunkArgs a) {
  __shared__ BucketLds bs;  // the last workgroup's tile layout
  __shared__ int s_wsum[4];
  __shared__ int s_last;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nwg = (a.T + kTopkBucketWaves - 1) / kTopkBucketWaves;
  int* const row = a.wg_cnt + (size_t)blockIdx.x * nwg;  // expert blockIdx.x
  const int per = (nwg + 255) / 256;
  const int i0 = min(nwg, (int)threadIdx.x * per), i1 = min(nwg, i0 + per);
  int sum = 0;
  for (int i = i0; i < i1; ++i) sum += row[i];
  int inc = sum;
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(inc, d, 64);
    if (lane >= d) inc += u;
  }
  if (lane == 63) s_wsum[wave] = inc;
  if (threadIdx.x < kTileClasses) bs.cls[0][threadIdx.x] = 0;
  __syncthreads();
  int base = inc - sum;
  for (int w2 = 0; w2 < wave; ++w2) base += s_wsum[w2];
  for (int i = i0; i < i1; ++i) {
    const int c = row[i];
    row[i] = base;
    base += c;
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(a.exp_cnt + blockIdx.x, s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are acknowledged
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(a.route_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x == 0) __hip_atomic_store(a.route_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  bucket_tiles(a, bs, [&](int e) { return e < a.E ? load_id<true>(a.exp_cnt + e) : 0; });
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) a.exp_off[e] = bs.off[e];
}

__global__ __launch_bounds__(64) void bucket_scatter_kernel(ChunkArgs a) {
  __shared__ int rank[kMaxExperts];
  const int lane = threadIdx.x;
  for (int i = lane; i < kMaxExperts; i += 64) rank[i] = 0;
  __builtin_amdgcn_wave_barrier();  // (one wave: its LDS operations complete in order)
  const int P = a.T * a.k;
  const int p0 = blockIdx.x * kTopkBucketWaves * a.k, p1 = min(P, p0 + kTopkBucketWaves * a.k);
  constexpr int kB = kTopkBucketWaves * kMaxTopK / 64;  // 64-pair batches of one top-k workgroup
  int ev[kB];
  float wv[kB];
#pragma unroll
  for (int u = 0; u < kB; ++u) {
    const int p = min(p0 + 64 * u + lane, P - 1);
    ev[u] = a.ids[p];
    wv[u] = a.wts[p];
  }
#pragma unroll
  for (int u = 0; u < kB; ++u) {
    const int p = p0 + 64 * u + lane, e = ev[u];
    if (p < p1 && e >= 0 && e < a.E) {
      const int pos = a.exp_off[e] + a.wg_cnt[(size_t)e * gridDim.x + blockIdx.x] + atomicAdd(&rank[e], 1);
      a.sorted_pair[pos] = p;
      a.sorted_wt[pos] = wv[u];
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped-GEMM tile core: acc[mt][f] += A[32*MT][K] . W_f[32][K]^T.
//
// A (activation rows) goes through LDS in stages of kKS = 128 (two 64-groups),
// double-buffered: the next stage's rows are loaded into registers while the
// current one is multiplied.  Each wave streams its own weight rows straight
// into registers one stage ahead.  The binary16 scale of each 64-group is
// folded into the weight conversion (code * scale rounded to binary16).
//
// All global reads are buffer loads through range-checked resources: a masked
// row or column gets an offset outside the resource and reads zeros, so no
// load sits under a branch or feeds a select (either would make the compiler
// wait for the load where it is issued instead of where it is used).
// ---------------------------------------------------------------------------
static constexpr int kKS = 128;
static constexpr int kAStride = kKS + 8;       // halves per LDS row (padding against bank conflicts)
// Weight stages in flight in the 32-row-block path, by row blocks: a tile with
// fewer rows has less MFMA work per stage to cover a weight fetch with, and
// smaller accumulators, which leave registers for more stages (128-row tiles
// have no registers for a second one).
__host__ __device__ constexpr int tile_pf(int mt) { return mt >= 3 ? 1 : (mt == 2 ? 2 : 3); }

template <int MT>
struct AStage {
  static constexpr int CH = kKS / 8;            // 16-byte chunks per row per stage
  static constexpr int N = 32 * MT * CH / 256;  // chunks per thread
  u32x4 v[N];
  // kbyte: byte offset of the stage in a row (kOob past the last stage)
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t res, const uint32_t off[N], uint32_t kbyte) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = ((int)threadIdx.x + 256 * i) % CH;
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(res, off[i] + kbyte + 16u * c, 0, 0);
    }
  }
  __device__ __forceinline__ void store(_Float16* lds) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = (int)threadIdx.x + 256 * i;
      const int m = idx / CH, c = idx % CH;
      *reinterpret_cast<h8*>(lds + m * kAStride + 8 * c) = act_operand(v[i]);
    }
  }
};

template <int BITS, int NF, bool AFF = false>
struct BStage {
  static constexpr int Q = BITS == 4 ? 1 : 2;  // 16-byte loads per lane per group
  u32x4 q[2][NF][Q];
  // qoff: byte offset of the lane's K slice in its weight row (kOob for a
  // masked row).  kb: first K of the stage; live = false turns every load into
  // an out-of-range one.
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rq, const uint32_t qoff[NF], int kb, bool live) {
    const uint32_t qk = live ? (uint32_t)kb * BITS / 8 : kOob;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int j = 0; j < Q; ++j)
          q[gi][f][j] = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff[f] + qk + (uint32_t)(kGroup * gi * BITS / 8 + 16 * j), 0, 0);
  }
  // MFMA operand for step st of group gi, fragment f; sw holds the binary16
  // scales of the stage's two groups (group gi in half gi), ow their offsets
  // (AFF: unsigned codes, w = q s + b)
  __device__ __forceinline__ h8 operand(int gi, int f, int st, uint32_t sw, uint32_t ow) const {
    h2 w[4];
    const uint32_t sel = gi ? 0x07060706u : 0x05040504u;
    const h2 sc = as_h2(__builtin_amdgcn_perm(sw, sw, sel));
    if (AFF) {
      uint4x8_to_h2x4(q[gi][f][0][st], w);
      const h2 bo = as_h2(__builtin_amdgcn_perm(ow, ow, sel));
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = __builtin_elementwise_fma(w[i], sc, bo);
      return pack8(w);
    }
    if (BITS == 4) {
      int4x8_to_h2x4(q[gi][f][0][st], w);
    } else {
      int8x8_to_h2x4(q[gi][f][st >> 1][2 * (st & 1)], q[gi][f][st >> 1][2 * (st & 1) + 1], w);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] *= sc;
    return pack8(w);
  }
};

// Scales of 8 consecutive groups (4 stages) of each fragment's weight row: one
// 16-byte load per fragment every 4 stages, instead of one 2-byte load per
// group and fragment.  Word j covers stage j of the block.
template <int NF>
struct ScaleBlock {
  u32x4 v[NF];
  // soff: byte offset of the row's scales (kOob for a masked row); blk: block
  // index (8 groups); live = false reads zeros.  Only for rows of at least 8
  // groups, so the 16 bytes lie inside the row and are 16-byte aligned in it.
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, const uint32_t soff[NF], int blk, bool live) {
    const uint32_t sk = live ? 16u * blk : kOob;
#pragma unroll
    for (int f = 0; f < NF; ++f) v[f] = __builtin_amdgcn_raw_buffer_load_b128(rs, soff[f] + sk, 0, 0);
  }
  // first block of a row of ng groups: a row shorter than 8 groups (ng = 1, 2
  // or 4) is read with a load of its own size, so no load reaches past the
  // row (or past the end of the tensor for the last row)
  __device__ __forceinline__ void load_first(__amdgpu_buffer_rsrc_t rs, const uint32_t soff[NF], int ng) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (ng >= 8) {
        v[f] = __builtin_amdgcn_raw_buffer_load_b128(rs, soff[f], 0, 0);
      } else if (ng == 4) {
        const auto d = __builtin_amdgcn_raw_buffer_load_b64(rs, soff[f], 0, 0);
        v[f] = u32x4{d[0], d[1], 0u, 0u};
      } else if (ng == 2) {
        v[f] = u32x4{__builtin_amdgcn_raw_buffer_load_b32(rs, soff[f], 0, 0), 0u, 0u, 0u};
      } else {
        v[f] = u32x4{(uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, soff[f], 0, 0), 0u, 0u, 0u};
      }
    }
  }
};

// Operands of one tile: A rows through `ra` at byte offsets aoff (one per
// 16-byte chunk this thread stages), weight fragments through rq/rs (and the
// offsets of affine weights through rb, laid out like the scales).
template <int BITS, int NF, int MT>
struct GemmOperands {
  __amdgpu_buffer_rsrc_t ra, rq, rs, rb;
  uint32_t aoff[AStage<MT>::N];
  uint32_t qoff[NF], soff[NF];
};

template <int BITS, int NF, int MT, bool AFF>
__device__ __forceinline__ void stage_mfma(const _Float16* L, const BStage<BITS, NF, AFF>& b, const uint32_t sw[NF],
                                           const uint32_t ow[NF], int kb, int K, f16v acc[MT][NF]) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 31, g = lane >> 5;
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    if (kb + kGroup * gi < K) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        h8 av[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          av[mt] = *reinterpret_cast<const h8*>(L + (32 * mt + m) * kAStride + kGroup * gi + 32 * g + 8 * s);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const h8 bv = b.operand(gi, f, s, sw[f], ow[f]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[mt], bv, acc[mt][f], 0, 0, 0);
        }
      }
    }
  }
}

template <int BITS, int NF, int MT, bool AFF = false>
__device__ __forceinline__ void tile_gemm(_Float16* lds, const GemmOperands<BITS, NF, MT>& op, int K,
                                          f16v acc[MT][NF]) {
  constexpr int BUF = 32 * MT * kAStride;
  constexpr int PF = tile_pf(MT);  // weight stages in flight
  static_assert(PF >= 1 && PF <= 3, "the stage ring holds four stages");
  const int nst = (K + kKS - 1) / kKS;
  AStage<MT> as;
  BStage<BITS, NF, AFF> b[4];
  ScaleBlock<NF> sc, scn, oc, ocn;  // scales, offsets (AFF)
  as.load(op.ra, op.aoff, 0);
#pragma unroll
  for (int i = 0; i < PF; ++i) b[i].load(op.rq, op.qoff, i * kKS, i < nst);
  sc.load_first(op.rs, op.soff, K / kGroup);
  if (AFF) oc.load_first(op.rb, op.soff, K / kGroup);
  as.store(lds);
  __syncthreads();
  // Four stages per iteration: stage s multiplies ring slot s % 4 and loads
  // the weights of stage s + PF into slot (s + PF) % 4; each iteration uses
  // one scale block, whose successor is loaded with the last stage's
  // prefetch.  The next stage's loads are issued unconditionally (out of
  // range past the last stage): loads issued on one path only would make the
  // compiler drain the load queue where the paths join.
#define MOE_TILE_STAGE(J, LC, LN)                                              \
  {                                                                            \
    const int kb = (st + J) * kKS;                                             \
    const bool more = st + J + 1 < nst;                                        \
    as.load(op.ra, op.aoff, more ? 2u * (kb + kKS) : kOob);                    \
    b[(J + PF) & 3].load(op.rq, op.qoff, kb + PF * kKS, st + J + PF < nst);   \
    if (J == 3) scn.load(op.rs, op.soff, st / 4 + 1, st + 4 < nst);            \
    if (AFF && J == 3) ocn.load(op.rb, op.soff, st / 4 + 1, st + 4 < nst);     \
    /* keep the next stage's loads ahead of this stage's arithmetic */         \
    __builtin_amdgcn_sched_barrier(0);                                         \
    uint32_t sw[NF], ow[NF];                                                   \
    _Pragma("unroll") for (int f = 0; f < NF; ++f) {                           \
      sw[f] = sc.v[f][J];                                                      \
      ow[f] = AFF ? oc.v[f][J] : 0u;                                           \
    }                                                                          \
    stage_mfma<BITS, NF, MT, AFF>(LC, b[J], sw, ow, kb, K, acc);               \
    as.store(LN);                                                              \
    __syncthreads();                                                           \
    if (!more) break;                                                          \
  }
  for (int st = 0; st < nst; st += 4) {
    MOE_TILE_STAGE(0, lds, lds + BUF)
    MOE_TILE_STAGE(1, lds + BUF, lds)
    MOE_TILE_STAGE(2, lds, lds + BUF)
    MOE_TILE_STAGE(3, lds + BUF, lds)
    sc = scn;
    if (AFF) oc = ocn;
  }
#undef MOE_TILE_STAGE
}

// LDS of one GEMM workgroup: two A buffers of kTileRows rows, or the rows
// of a narrow tile for the whole K (below)
static constexpr int kNarrowStride = kNarrowK + 8;  // halves per LDS row of a narrow tile
static constexpr int kGemmLds = 2 * kTileRows * kAStride > kNarrowRows * kNarrowStride
                                    ? 2 * kTileRows * kAStride : kNarrowRows * kNarrowStride;

struct TileRows {
  uint32_t aoff[kTileRows];  // byte offset of each A row in its resource (kOob: zero row)
  int out_row[kTileRows];    // destination row
  float scale[kTileRows];    // epilogue scale (routing weight or sigma)
};

template <int BITS, int NF, int MT>
__device__ __forceinline__ void set_a_offsets(GemmOperands<BITS, NF, MT>& op, const TileRows& tr) {
#pragma unroll
  for (int i = 0; i < AStage<MT>::N; ++i) op.aoff[i] = tr.aoff[((int)threadIdx.x + 256 * i) / AStage<MT>::CH];
}

// ---------------------------------------------------------------------------
// Narrow tiles (at most kNarrowRows rows, K a power of two in [kNarrowMinK,
// kNarrowK]): the tile's
// activation rows stay in LDS for the whole K, and each wave streams its own
// weight rows kNarrowPF stages ahead with no workgroup barrier inside the K
// loop.  MFMA 16x16x32 f16: lane l = 16q + n works on row n of each 16-row
// operand, and in MFMA step t of a 128-K stage on K = 32q + 8t .. +8 (the
// same for activations and weights, so the products pair up).  A lane's int4
// weights of one stage are then 16 contiguous bytes of its row: one load per
// fragment and stage, four lanes per 64-byte run of a row.  Accumulator
// element i of lane l is row 4q + i, column n.
// ---------------------------------------------------------------------------
static constexpr int kNarrowMinK = 512;             // one scale block per row at least
static constexpr int kNarrowPF = 2;                  // weight stages in flight

// the tile's activation rows for K in [0, 128 N): N 16-byte chunks per thread
template <int N>
struct NarrowA {
  u32x4 v[N];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t ra, const uint32_t* aoff, int K) {
    constexpr int CPR = N * 256 / kNarrowRows;  // 16-byte chunks per row
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = (int)threadIdx.x + 256 * i;
      const int row = c / CPR, col = c % CPR;
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, 8 * col < K ? aoff[row] + 16u * col : kOob, 0, 0);
    }
  }
  __device__ __forceinline__ void store(_Float16* lds) const {
    constexpr int CPR = N * 256 / kNarrowRows;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = (int)threadIdx.x + 256 * i;
      *reinterpret_cast<h8*>(lds + (c / CPR) * kNarrowStride + 8 * (c % CPR)) = act_operand(v[i]);
    }
  }
};

// One stage of int4 weights: 16 bytes (32 K) per lane and fragment.  The
// loads are coalesced (lane l reads part l % 4 of row l / 4 of the
// fragment's 64-byte stage run, so four neighbouring lanes cover one run) and
// the bytes are then moved to the MFMA lane (row l % 16, part l / 16) with a
// cross-lane permute: neighbouring lanes reading different rows would make
// the texture addresser take the lanes one by one.
template <int NF>
struct NarrowB {
  u32x4 q[NF];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rq, const uint32_t qoff[NF], int st, bool live) {
    const uint32_t k = live ? 64u * st : kOob;
#pragma unroll
    for (int f = 0; f < NF; ++f) q[f] = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff[f] + k, 0, 0);
  }
};

// the 16 bytes that the coalesced load gave lane 4 (l % 16) + l / 16, in lane l
__device__ __forceinline__ u32x4 to_mfma_lanes(u32x4 v, int src_byte) {
  u32x4 r;
  r.x = (uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)v.x);
  r.y = (uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)v.y);
  r.z = (uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)v.z);
  r.w = (uint32_t)__builtin_amdgcn_ds_bpermute(src_byte, (int)v.w);
  return r;
}

template <int N, int NF>
__device__ __forceinline__ void narrow_prologue(_Float16* lds, __amdgpu_buffer_rsrc_t ra, const uint32_t* aoff, int K,
                                                __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rs,
                                                const uint32_t qoff[NF], const uint32_t soff[NF], NarrowB<NF> b[4],
                                                ScaleBlock<NF>& sc, int nst) {
  NarrowA<N> a;
  a.load(ra, aoff, K);  // activations first: their store below waits for them alone
  sc.load(rs, soff, 0, true);  // K >= 512: a whole block of 8 groups
#pragma unroll
  for (int i = 0; i < kNarrowPF; ++i) b[i].load(rq, qoff, i, i < nst);
  a.store(lds);
}

// acc[f] += A[16][K] . W_f[16][K]^T for the wave's NF weight fragments (AFF:
// unsigned codes and offsets through rb, laid out like the scales)
template <int NF, bool AFF = false>
__device__ __forceinline__ void narrow_gemm(_Float16* lds, __amdgpu_buffer_rsrc_t ra, const uint32_t* aoff, int K,
                                            __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rs,
                                            __amdgpu_buffer_rsrc_t rb, const uint32_t qoff[NF],
                                            const uint32_t soff[NF], f4 acc[NF]) {
  static_assert(kNarrowPF >= 1 && kNarrowPF <= 3, "the stage ring holds four stages");
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const uint32_t ssel = (q & 2) ? 0x07060706u : 0x05040504u;  // the lane's group in the stage: half q/2 of a scale word
  const int src_byte = 4 * (4 * n + q);                          // coalesced lane holding this lane's weights
  const int nst = (K + kKS - 1) / kKS;
  NarrowB<NF> b[4];
  ScaleBlock<NF> sc, scn, oc, ocn;
  // K is a multiple of 512 here, so the K loop runs whole iterations of four
  // stages with no exit inside one: every path into the loop head has issued
  // the same loads, and the compiler's wait counts keep kNarrowPF stages in
  // flight.
  switch (nst) {
    case 4: narrow_prologue<4, NF>(lds, ra, aoff, K, rq, rs, qoff, soff, b, sc, nst); break;
    case 8: narrow_prologue<8, NF>(lds, ra, aoff, K, rq, rs, qoff, soff, b, sc, nst); break;
    default: narrow_prologue<16, NF>(lds, ra, aoff, K, rq, rs, qoff, soff, b, sc, nst); break;
  }
  if (AFF) oc.load(rb, soff, 0, true);
  __syncthreads();
  const _Float16* La = lds + n * kNarrowStride + 32 * q;
  // Four stages per iteration (one scale block): stage s computes from ring
  // slot s % 4 and loads stage s + kNarrowPF into slot (s + kNarrowPF) % 4.
#define MOE_NARROW_STAGE(J)                                                                \
  {                                                                                        \
    const int s_ = st + J;                                                                 \
    b[(J + kNarrowPF) & 3].load(rq, qoff, s_ + kNarrowPF, s_ + kNarrowPF < nst);           \
    if (J == 0) scn.load(rs, soff, st / 4 + 1, st + 4 < nst);                              \
    if (AFF && J == 0) ocn.load(rb, soff, st / 4 + 1, st + 4 < nst);                       \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    h2 scl[NF], ofl[NF];                                                                   \
    u32x4 bw[NF];                                                                          \
    _Pragma("unroll") for (int f = 0; f < NF; ++f) {                                       \
      scl[f] = as_h2(__builtin_amdgcn_perm(sc.v[f][J], sc.v[f][J], ssel));                 \
      ofl[f] = AFF ? as_h2(__builtin_amdgcn_perm(oc.v[f][J], oc.v[f][J], ssel)) : scl[f]; \
      bw[f] = to_mfma_lanes(b[J].q[f], src_byte);                                          \
    }                                                                                      \
    _Pragma("unroll") for (int t = 0; t < 4; ++t) {                                        \
      const h8 av = *reinterpret_cast<const h8*>(La + kKS * s_ + 8 * t);                  \
      _Pragma("unroll") for (int f = 0; f < NF; ++f) {                                     \
        h2 w[4];                                                                           \
        if (AFF) {                                                                         \
          uint4x8_to_h2x4(bw[f][t], w);                                                    \
          _Pragma("unroll") for (int i = 0; i < 4; ++i)                                    \
            w[i] = __builtin_elementwise_fma(w[i], scl[f], ofl[f]);                        \
        } else {                                                                           \
          int4x8_to_h2x4(bw[f][t], w);                                                     \
          _Pragma("unroll") for (int i = 0; i < 4; ++i) w[i] *= scl[f];                    \
        }                                                                                  \
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pack8(w), acc[f], 0, 0, 0);    \
      }                                                                                    \
    }                                                                                      \
  }
  for (int st = 0; st < nst; st += 4) {
    MOE_NARROW_STAGE(0)
    MOE_NARROW_STAGE(1)
    MOE_NARROW_STAGE(2)
    MOE_NARROW_STAGE(3)
    sc = scn;
    if (AFF) oc = ocn;
  }
#undef MOE_NARROW_STAGE
}

// ---------------------------------------------------------------------------
// Work order.  Tiles are listed heaviest first.  Item r is (tile, column
// block) with the tiles taken in groups of 8: inside a group the 8 tiles of
// one column block are consecutive, so r % 8 = tile % 8.  The dispatcher
// hands block b to XCD b % 8; with C compute units and two GEMM workgroups
// per unit, blocks 0..C-1 start one per unit and block C + i takes the second
// slot of block i's unit.  Block b < C takes item b; block C + i takes the
// item i'-th from the end, where i' reverses i inside its group of 8, so each
// unit pairs a heavy item with a light one and every item of a tile runs on
// XCD tile % 8 (one L2 holds the tile's activation rows).  Blocks from 2C on
// take the middle of the list as slots free up.  For any C the map is
// one-to-one onto the n items (n a multiple of 8); for C not a multiple of 8
// the reversal is dropped.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int paired_item(int n_items, int cus) {
  const int b = blockIdx.x;
  int r;
  if (b < cus) {
    r = b;
  } else if (b < 2 * cus) {
    const int i = b - cus;
    r = n_items - 1 - (cus % 8 == 0 ? (i & ~7) | (7 - (i & 7)) : i);
    if (r < cus) return -1;
  } else {
    r = b - cus;
    if (r >= n_items - cus) return -1;
  }
  return r < n_items ? r : -1;
}

// item r of nb column blocks per tile -> (tile, column block)
__device__ __forceinline__ void item_of(int r, int nb, int& tile, int& cb) {
  const int g = r / (8 * nb), rem = r - g * 8 * nb;
  cb = rem >> 3;
  tile = 8 * g + (rem & 7);
}

// ---------------------------------------------------------------------------
// 4. gate/up GEMM with SwiGLU epilogue.  Items: (column block of 128, tile),
//    column-block major; routed tiles first, then shared-expert tiles.
// ---------------------------------------------------------------------------
template <int BITS, int MT, bool AFF = false>
__device__ __forceinline__ void up_tile(const ChunkArgs& a, _Float16* lds, const TileRows& tr,
                                        __amdgpu_buffer_rsrc_t ra, const uint8_t* wq, const uint16_t* wsc,
                                        const uint16_t* wof, int inter, int jb, _Float16* hout, int rows) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = jb * 128 + wave * 32 + (lane & 31);
  const uint32_t rb = (uint32_t)a.H * BITS / 8;
  const uint32_t ng = a.H / kGroup;
  const bool ok = j < inter;
  GemmOperands<BITS, 2, MT> op;
  op.ra = ra;
  op.rq = make_rsrc(wq, 2u * inter * rb);
  op.rs = make_rsrc(wsc, 2u * inter * ng * 2u);
  if (AFF) op.rb = make_rsrc(wof, 2u * inter * ng * 2u);
  const uint32_t kl = 32u * (lane >> 5) * BITS / 8;  // the lane's K slice inside a group
  op.qoff[0] = ok ? (uint32_t)j * rb + kl : kOob;
  op.qoff[1] = ok ? (uint32_t)(inter + j) * rb + kl : kOob;
  op.soff[0] = ok ? (uint32_t)j * ng * 2u : kOob;
  op.soff[1] = ok ? (uint32_t)(inter + j) * ng * 2u : kOob;
  set_a_offsets(op, tr);
  f16v acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt][0] = acc[mt][1] = f16v{};
  tile_gemm<BITS, 2, MT, AFF>(lds, op, a.H, acc);  // ends with a workgroup barrier: the LDS is free
  // The wave's h tile goes through LDS (row-major, 32 halves a row) so that
  // the stores are whole 16-byte pieces of rows, not one 2-byte value a lane.
  _Float16* ht = lds + wave * (32 * MT) * 32;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      ht[(32 * mt + acc_row(i)) * 32 + (lane & 31)] = (_Float16)(silu_f(acc[mt][0][i]) * acc[mt][1][i]);
  __syncthreads();
  if (jb * 128 + wave * 32 >= inter) return;  // widths are multiples of 64: a wave's columns are all in or all out
  const int c = lane & 3;
  for (int r = lane >> 2; r < rows; r += 16)
    *reinterpret_cast<uint4*>(hout + (size_t)tr.out_row[r] * inter + jb * 128 + wave * 32 + 8 * c) =
        *reinterpret_cast<const uint4*>(ht + r * 32 + 8 * c);
}

// a narrow routed tile: each wave takes 32 gate and the same 32 up columns as
// four 16-column fragments (gate j0.., gate j0+16.., up j0.., up j0+16..)
template <bool AFF>
__device__ __forceinline__ void up_narrow(const ChunkArgs& a, _Float16* lds, const TileRows& tr,
                                          __amdgpu_buffer_rsrc_t ra, const uint8_t* wq, const uint16_t* wsc,
                                          const uint16_t* wof, int inter, int jb, _Float16* hout, int rows) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const uint32_t rb = (uint32_t)a.H / 2;
  const uint32_t ng = a.H / kGroup;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(wq, 2u * inter * rb);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(wsc, 2u * inter * ng * 2u);
  const __amdgpu_buffer_rsrc_t ro = AFF ? make_rsrc(wof, 2u * inter * ng * 2u) : rs;
  const int j0 = jb * 128 + wave * 32;
  uint32_t qoff[4], soff[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int j = j0 + 16 * (f & 1) + n;              // the MFMA lane's column (scales)
    const int jl = j0 + 16 * (f & 1) + (lane >> 2);   // the row this lane loads (weights)
    qoff[f] = jl < inter ? (uint32_t)((f >> 1) * inter + jl) * rb + 16u * (lane & 3) : kOob;
    soff[f] = j < inter ? (uint32_t)((f >> 1) * inter + j) * ng * 2u : kOob;
  }
  f4 acc[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) acc[f] = f4{0.f, 0.f, 0.f, 0.f};
  narrow_gemm<4, AFF>(lds, ra, tr.aoff, a.H, rq, rs, ro, qoff, soff, acc);
  // h through LDS (16 rows of 32 halves per wave) for 16-byte row stores;
  // the barrier first: other waves may still read the tile's rows
  __syncthreads();
  _Float16* ht = lds + wave * kNarrowRows * 32;
#pragma unroll
  for (int ff = 0; ff < 2; ++ff)
#pragma unroll
    for (int i = 0; i < 4; ++i) ht[(4 * q + i) * 32 + 16 * ff + n] = (_Float16)(silu_f(acc[ff][i]) * acc[ff + 2][i]);
  __syncthreads();
  const int r = lane >> 2, c = lane & 3;
  if (j0 < inter && r < rows)
    *reinterpret_cast<uint4*>(hout + (size_t)tr.out_row[r] * inter + j0 + 8 * c) =
        *reinterpret_cast<const uint4*>(ht + r * 32 + 8 * c);
}

template <bool AFF>
__global__ __launch_bounds__(256, 2) void up_gemm_kernel(ChunkArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[kGemmLds];
  __shared__ TileRows tr;
  // items: (tile, column block of 128) over the cost-ordered tiles
  const int nbi = (a.I + 127) / 128, nbs = (a.Is + 127) / 128, nbm = max(nbi, nbs);
  const int nt = *a.n_tiles;
  const int w = paired_item(((nt + 7) & ~7) * nbm, a.cus);
  if (w < 0) return;
  int tile, jb;
  item_of(w, nbm, tile, jb);
  if (tile >= nt) return;
  const int4 td = a.tiles[tile];
  const int e = td.x, r0 = td.y, rows = td.z, mt = td.w;
  if (jb >= (e >= 0 ? nbi : nbs)) return;
  if (threadIdx.x < kTileRows) {
    const int r = threadIdx.x;
    int tok = -1;
    if (e >= 0) {
      const int p = r < rows ? a.sorted_pair[r0 + r] : -1;
      tok = p >= 0 ? p / a.k : -1;
    } else if (r < rows) {
      tok = r0 + r;
    }
    tr.aoff[r] = tok >= 0 ? (uint32_t)tok * a.H * 2u : kOob;
    tr.out_row[r] = r0 + r;
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.xa, (uint32_t)a.T * a.H * 2u);
  if (e >= 0) {
    const uint8_t* wq = a.w13_q + (size_t)e * 2 * a.I * (a.H / 2);
    const size_t so = (size_t)e * 2 * a.I * (a.H / kGroup);
    const uint16_t* wsc = a.w13_s + so;
    const uint16_t* wof = AFF ? a.w13_b + so : nullptr;
    switch (mt) {
      case 4:
        if constexpr (kTileRows >= 128) {
          up_tile<4, 4, AFF>(a, lds, tr, ra, wq, wsc, wof, a.I, jb, a.h, rows);
          break;
        }
        [[fallthrough]];
      case 3: up_tile<4, 3, AFF>(a, lds, tr, ra, wq, wsc, wof, a.I, jb, a.h, rows); break;
      case 2: up_tile<4, 2, AFF>(a, lds, tr, ra, wq, wsc, wof, a.I, jb, a.h, rows); break;
      case 0:
        if (a.H >= kNarrowMinK && a.H <= kNarrowK) {
          up_narrow<AFF>(a, lds, tr, ra, wq, wsc, wof, a.I, jb, a.h, rows);
          break;
        }
        [[fallthrough]];
      default: up_tile<4, 1, AFF>(a, lds, tr, ra, wq, wsc, wof, a.I, jb, a.h, rows); break;
    }
  } else {
    const uint8_t* wq = reinterpret_cast<const uint8_t*>(a.sh13_q);
    if (mt == 2) up_tile<8, 2>(a, lds, tr, ra, wq, a.sh13_s, nullptr, a.Is, jb, a.hs, rows);
    else up_tile<8, 1>(a, lds, tr, ra, wq, a.sh13_s, nullptr, a.Is, jb, a.hs, rows);
  }
}

// ---------------------------------------------------------------------------
// 5. down GEMM: y[row][n] = w_row * (h_row . W_down[n]); shared tiles write
//    ys[t][n] = sigma_t * (h_s[t] . S_down[n]).  Items: (block of 256
//    outputs, tile), output-block major.
// ---------------------------------------------------------------------------
// The destination row and scale of tile row threadIdx.x (< kTileRows) come
// in registers (my_row, my_scale): they were loaded before the K loop and
// are published to the TileRows of the epilogue after it, so their loads
// never delay the GEMM.
__device__ __forceinline__ void publish_rows(TileRows& tr, int my_row, float my_scale) {
  if (threadIdx.x < kTileRows) {
    tr.out_row[threadIdx.x] = my_row;
    tr.scale[threadIdx.x] = my_scale;
  }
}

template <int BITS, int MT, bool AFF = false>
__device__ __forceinline__ void down_tile(const ChunkArgs& a, _Float16* lds, TileRows& tr,
                                          __amdgpu_buffer_rsrc_t ra, const uint8_t* wq, const uint16_t* wsc,
                                          const uint16_t* wof, int K, int nb, _Float16* yout, int rows, int my_row,
                                          float my_scale) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t rb = (uint32_t)K * BITS / 8;
  const uint32_t ng = K / kGroup;
  GemmOperands<BITS, 2, MT> op;
  op.ra = ra;
  op.rq = make_rsrc(wq, (uint32_t)a.H * rb);
  op.rs = make_rsrc(wsc, (uint32_t)a.H * ng * 2u);
  if (AFF) op.rb = make_rsrc(wof, (uint32_t)a.H * ng * 2u);
  const uint32_t kl = 32u * (lane >> 5) * BITS / 8;
  int n[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    n[f] = nb * 256 + wave * 64 + f * 32 + (lane & 31);
    const bool ok = n[f] < a.H;
    op.qoff[f] = ok ? (uint32_t)n[f] * rb + kl : kOob;
    op.soff[f] = ok ? (uint32_t)n[f] * ng * 2u : kOob;
  }
  set_a_offsets(op, tr);
  f16v acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt][0] = acc[mt][1] = f16v{};
  tile_gemm<BITS, 2, MT, AFF>(lds, op, K, acc);  // ends with a workgroup barrier: the LDS is free
  publish_rows(tr, my_row, my_scale);
  __syncthreads();
  // the wave's 64 outputs of each row through LDS (row-major, 64 halves a
  // row) for 16-byte row stores
  _Float16* yt = lds + wave * (32 * MT) * 64;
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 32 * mt + acc_row(i);
        yt[r * 64 + 32 * f + (lane & 31)] = (_Float16)(tr.scale[r] * acc[mt][f][i]);
      }
  __syncthreads();
  const int c0 = nb * 256 + wave * 64;
  if (c0 >= a.H) return;  // H is a multiple of 64: a wave's outputs are all in or all out
  const int c = lane & 7;
  for (int r = lane >> 3; r < rows; r += 8)
    *reinterpret_cast<uint4*>(yout + (size_t)tr.out_row[r] * a.H + c0 + 8 * c) =
        *reinterpret_cast<const uint4*>(yt + r * 64 + 8 * c);
}

// a narrow routed tile: each wave takes 64 outputs as four 16-column fragments
template <bool AFF>
__device__ __forceinline__ void down_narrow(const ChunkArgs& a, _Float16* lds, TileRows& tr,
                                            __amdgpu_buffer_rsrc_t ra, const uint8_t* wq, const uint16_t* wsc,
                                            const uint16_t* wof, int K, int nb, _Float16* yout, int rows, int my_row,
                                            float my_scale) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const uint32_t rb = (uint32_t)K / 2;
  const uint32_t ng = K / kGroup;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(wq, (uint32_t)a.H * rb);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(wsc, (uint32_t)a.H * ng * 2u);
  const __amdgpu_buffer_rsrc_t ro = AFF ? make_rsrc(wof, (uint32_t)a.H * ng * 2u) : rs;
  int col[4];
  uint32_t qoff[4], soff[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    col[f] = nb * 256 + wave * 64 + 16 * f + n;             // the MFMA lane's column (scales, output)
    const int cl = nb * 256 + wave * 64 + 16 * f + (lane >> 2);  // the row this lane loads (weights)
    qoff[f] = cl < a.H ? (uint32_t)cl * rb + 16u * (lane & 3) : kOob;
    soff[f] = col[f] < a.H ? (uint32_t)col[f] * ng * 2u : kOob;
  }
  f4 acc[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) acc[f] = f4{0.f, 0.f, 0.f, 0.f};
  narrow_gemm<4, AFF>(lds, ra, tr.aoff, K, rq, rs, ro, qoff, soff, acc);
  // outputs through LDS (16 rows of 64 halves per wave) for 16-byte row
  // stores; the barrier first: other waves may still read the tile's rows
  publish_rows(tr, my_row, my_scale);
  __syncthreads();
  _Float16* yt = lds + wave * kNarrowRows * 64;
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) yt[(4 * q + i) * 64 + 16 * f + n] = (_Float16)(tr.scale[4 * q + i] * acc[f][i]);
  __syncthreads();
  const int c0 = nb * 256 + wave * 64;
  if (c0 >= a.H) return;
  const int c = lane & 7;
#pragma unroll
  for (int r = lane >> 3; r < kNarrowRows; r += 8)
    if (r < rows)
      *reinterpret_cast<uint4*>(yout + (size_t)tr.out_row[r] * a.H + c0 + 8 * c) =
          *reinterpret_cast<const uint4*>(yt + r * 64 + 8 * c);
}

template <bool AFF>
__global__ __launch_bounds__(256, 2) void down_gemm_kernel(ChunkArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[kGemmLds];
  __shared__ TileRows tr;
  // items: (tile, block of 256 outputs) over the cost-ordered tiles
  const int nbh = (a.H + 255) / 256;
  const int nt = *a.n_tiles;
  const int w = paired_item(((nt + 7) & ~7) * nbh, a.cus);
  if (w < 0) return;
  int tile, nb;
  item_of(w, nbh, tile, nb);
  if (tile >= nt) return;
  const int4 td = a.tiles[tile];
  const int e = td.x, r0 = td.y, rows = td.z, mt = td.w;
  const int K = e >= 0 ? a.I : a.Is;
  // A is the tile's own rows of h (or h_s): its offsets need no loads.  The
  // destination row (routed rows of y are indexed by pair t * k + i, so the
  // combine reads a token's rows directly) and the scale of each row are
  // loaded now, with clamped indices, and used only in the epilogue.
  int my_row = 0;
  float my_scale = 0.f;
  if (threadIdx.x < kTileRows) {
    const int r = threadIdx.x, rc = r0 + min(r, rows - 1);
    if (e >= 0) {
      my_row = a.sorted_pair[rc];
      my_scale = a.sorted_wt[rc];
    } else {
      my_row = r0 + r;
      my_scale = a.sigma[rc];
    }
    tr.aoff[r] = r < rows ? (uint32_t)r * K * 2u : kOob;
  }
  __syncthreads();
  // A: the tile's own rows of h (or h_s), which start at row r0
  const _Float16* abase = (e >= 0 ? a.h : a.hs) + (size_t)r0 * K;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(abase, (uint32_t)rows * K * 2u);
  if (e >= 0) {
    const uint8_t* wq = a.w2_q + (size_t)e * a.H * (a.I / 2);
    const size_t so = (size_t)e * a.H * (a.I / kGroup);
    const uint16_t* wsc = a.w2_s + so;
    const uint16_t* wof = AFF ? a.w2_b + so : nullptr;
    switch (mt) {
      case 4:
        if constexpr (kTileRows >= 128) {
          down_tile<4, 4, AFF>(a, lds, tr, ra, wq, wsc, wof, a.I, nb, a.y, rows, my_row, my_scale);
          break;
        }
        [[fallthrough]];
      case 3: down_tile<4, 3, AFF>(a, lds, tr, ra, wq, wsc, wof, a.I, nb, a.y, rows, my_row, my_scale); break;
      case 2: down_tile<4, 2, AFF>(a, lds, tr, ra, wq, wsc, wof, a.I, nb, a.y, rows, my_row, my_scale); break;
      case 0:
        if (a.I >= kNarrowMinK && a.I <= kNarrowK) {
          down_narrow<AFF>(a, lds, tr, ra, wq, wsc, wof, a.I, nb, a.y, rows, my_row, my_scale);
          break;
        }
        [[fallthrough]];
      default: down_tile<4, 1, AFF>(a, lds, tr, ra, wq, wsc, wof, a.I, nb, a.y, rows, my_row, my_scale); break;
    }
  } else {
    const uint8_t* wq = reinterpret_cast<const uint8_t*>(a.sh2_q);
    if (mt == 2) down_tile<8, 2>(a, lds, tr, ra, wq, a.sh2_s, nullptr, a.Is, nb, a.ys, rows, my_row, my_scale);
    else down_tile<8, 1>(a, lds, tr, ra, wq, a.sh2_s, nullptr, a.Is, nb, a.ys, rows, my_row, my_scale);
  }
}

// ---------------------------------------------------------------------------
// 6. combine: out[t][n] = sum_i y[t*k+i][n] (+ ys[t][n]); 8 outputs/thread
// ---------------------------------------------------------------------------
__device__ __forceinline__ void add8(float acc[8], uint4 v) {
  const h8 h = __builtin_bit_cast(h8, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] += (float)h[i];
}

__global__ __launch_bounds__(256) void combine_kernel(ChunkArgs a) {
  // a one-dimensional grid of T x nbx blocks (a token's row is nbx blocks of
  // 2048 outputs), so T is not bound by the limit of a grid's second dimension
  const int nbx = (a.H / 8 + 255) / 256;
  const int t = blockIdx.x / nbx;
  const int n = ((blockIdx.x - t * nbx) * blockDim.x + threadIdx.x) * 8;
  if (n >= a.H) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // the token's k rows of y (row t * k + i) and its ids are loaded together;
  // a pair whose id is outside [0, E) was dropped and its row never written
  uint4 v[kMaxTopK];
  int id[kMaxTopK];
  const int i_last = (int)(((size_t)t + 1) * a.k - 1);
#pragma unroll
  for (int i = 0; i < kMaxTopK; ++i) {
    const int p = min(t * a.k + i, i_last);  // clamped: always a row of this token
    id[i] = a.ids[p];
    v[i] = *reinterpret_cast<const uint4*>(a.y + (size_t)p * a.H + n);
  }
  if (a.ys) add8(acc, *reinterpret_cast<const uint4*>(a.ys + (size_t)t * a.H + n));
  if (a.resid) add8(acc, *reinterpret_cast<const uint4*>(a.resid + (size_t)t * a.H + n));
#pragma unroll
  for (int i = 0; i < kMaxTopK; ++i)
    if (i < a.k && id[i] >= 0 && id[i] < a.E) add8(acc, v[i]);
  h8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (_Float16)acc[i];
  *reinterpret_cast<h8*>(a.out + (size_t)t * a.H + n) = o;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// the router GEMM with whole logits
static void launch_router_whole(const ChunkArgs& a, hipStream_t s) {
  if (a.T > kRouterRowsT && a.H / kGroup <= 4 * kRouterWaves)
    hipLaunchKernelGGL(router_rows_kernel, dim3((a.T + 31) / 32), dim3(64 * kRouterWaves), 0, s, a);
  else
    hipLaunchKernelGGL(router_gemm_kernel<4>, dim3((a.T + 31) / 32, (a.E + 1 + 31) / 32), dim3(64 * kRouterWaves), 0,
                       s, a);
}

int launch_route_chunk(const ChunkArgs& a0, hipStream_t s) {
  ChunkArgs a = a0;
  a.logits_hi = nullptr;  // whole logits: the caller may ask for them
  launch_router_whole(a, s);
  hipLaunchKernelGGL(topk_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

static void launch_gemms(const ChunkArgs& a, hipStream_t s);

int launch_experts_chunk(const ChunkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(1024), 0, s, a);
  launch_gemms(a, s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

int launch_forward_chunk(const ChunkArgs& a0, hipStream_t s) {
  // The router GEMM is split over K when its grid would be small (at most 64
  // workgroups: up to 224 tokens at 257 rows), except in the sub-block, whose
  // norm needs each workgroup to see whole rows.  (Measured: 1.3-1.6 us faster
  // at 32 and 128 tokens, 0.6 us slower at 512.)
  ChunkArgs a = a0;
  const int router_wgs = ((a.T + 31) / 32) * ((a.E + 1 + 31) / 32);
  if (a.gain || router_wgs > 64) a.logits_hi = nullptr;
  const int ks = a.logits_hi ? 2 : 1;
  if (ks == 2)
    hipLaunchKernelGGL(router_gemm_kernel<2>, dim3((a.T + 31) / 32, (a.E + 1 + 31) / 32, 2), dim3(64 * kRouterWaves), 0,
                       s, a);
  else
    launch_router_whole(a, s);
  // a few tokens per workgroup spread the ranking over more compute units,
  // while at most 64 workgroups (up to 1024 tokens) contend for the completion
  // counter, whose atomics are served one at a time
  if (a.T > kGridBucketT) {
    const int nwg = (a.T + kTopkBucketWaves - 1) / kTopkBucketWaves;
    hipLaunchKernelGGL(topk_count_kernel, dim3(nwg), dim3(64 * kTopkBucketWaves), 0, s, a);
    hipLaunchKernelGGL(bucket_scan_kernel, dim3(a.E), dim3(256), 0, s, a);
    hipLaunchKernelGGL(bucket_scatter_kernel, dim3(nwg), dim3(64), 0, s, a);
  } else {
    const int tpw = a.T <= 256 ? 4 : min(kTopkBucketWaves, max(4, (a.T + 63) / 64));
    hipLaunchKernelGGL(topk_bucket_kernel, dim3((a.T + tpw - 1) / tpw), dim3(64 * kTopkBucketWaves), 0, s, a);
  }
  launch_gemms(a, s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

static void launch_gemms(const ChunkArgs& a, hipStream_t s) {
  // grids over the item lists (tile count rounded up to a group of 8); blocks
  // beyond the items the bucketing produced exit at once
  const int max_tiles = (a.max_route_tiles + a.shared_tiles + 7) & ~7;
  const int up_items = max_tiles * max((a.I + 127) / 128, (a.Is + 127) / 128);
  const int down_items = max_tiles * ((a.H + 255) / 256);
  if (a.affine) {
    hipLaunchKernelGGL(up_gemm_kernel<true>, dim3((up_items + 7) & ~7), dim3(256), 0, s, a);
    hipLaunchKernelGGL(down_gemm_kernel<true>, dim3((down_items + 7) & ~7), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(up_gemm_kernel<false>, dim3((up_items + 7) & ~7), dim3(256), 0, s, a);
    hipLaunchKernelGGL(down_gemm_kernel<false>, dim3((down_items + 7) & ~7), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(combine_kernel, dim3((a.H / 8 + 255) / 256 * a.T), dim3(256), 0, s, a);
}

}  // namespace moe
