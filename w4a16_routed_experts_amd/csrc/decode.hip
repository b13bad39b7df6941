// Few-token path of the routed MoE block: one persistent launch.
//
// The block (the Chimera notebook, section 5): out = routed + sigmoid(x . W_sg)
// * shared, where the routed part is the renormalised top-k mixture of int4
// SwiGLU experts (section 5.2 ordering: softmax -> top-k -> renormalise) and
// the router rows are int8 group-64 rows stacked with the shared-gate row (the
// TensorFold PR, "Design").
//
// Work is split into items executed by a grid of co-resident workgroups.  Items
// hand results to each other through counters instead of kernel boundaries
// (one launch costs about as much as the whole layer's HBM time at one token):
//   A  router rows (logits) | shared-expert gate/up rows (h_s)
//   B  expert gate/up rows of the k selected experts (h_e, binary16)  <- router
//      shared-expert down rows (s)                           <- shared gate/up
//   C  expert down rows + weighted combine + sigma * s       <- B
// Every workgroup recomputes the top-k from the logits (one wave per token,
// see wave_topk), so no hand-off is needed between routing and the experts.  The
// weights of a workgroup's first C item are loaded before it waits.
//
// Hand-off without cache maintenance.  On gfx950 each XCD has its own L2, and
// agent-scope fences write back or invalidate a whole L2.  Instead:
//   * a producer writes its values with device-coherent stores into a region
//     of the workspace that only it writes (128-byte aligned, so no cache line
//     is shared between producers), waits until they are acknowledged
//     (vmcnt 0) and then bumps a counter with a device-scope atomic;
//   * a consumer polls the counter with device-coherent loads and then reads
//     the values with ordinary loads: no L2 can hold a stale copy, because the
//     L2s start each launch invalidated and nothing reads these lines before
//     their counter is complete.  The ordinary loads let each XCD's L2 serve
//     the many workgroups that read the same values.
#include "decode.hpp"
#include "gemv.hpp"

namespace moe {

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ void st_co(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_co_h(uint16_t* p, float v) {
  __hip_atomic_store(p, __builtin_bit_cast(uint16_t, (_Float16)v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Completion signalling.  Items of a stage count on kSubCounters
// sub-counters (item mod 8, each on its own 128-byte line) with device-scope
// atomics; the item that completes a sub-counter sets the sub-counter's bit
// in the stage's done word of each XCD's flag page.  Consumers poll only
// their own XCD's word (device-coherent loads) until every bit is set: no
// line is polled by more than one XCD's workgroups, the counters are never
// polled, and no counter takes more than about n/8 increments.
__device__ __forceinline__ int xcc_id() {
  return (int)(__builtin_amdgcn_s_getreg(20 | (15 << 11)) & (kXcds - 1));  // HW_REG_XCC_ID[3:0]
}
__device__ __forceinline__ uint32_t* counter_of(uint32_t* sync, int which, int sub) {
  return sync + (which * (kSubCounters + 1) + sub) * kSyncStride;
}
__device__ __forceinline__ uint32_t* flag_of(uint32_t* sync, int xcd, int which) {
  return sync + (kCounterPages + xcd) * kFlagPage + which * kSyncStride;
}
// done word of a stage of n items: one bit per non-empty sub-counter
__device__ __forceinline__ uint32_t done_mask(int n) { return (1u << (n < kSubCounters ? n : kSubCounters)) - 1u; }

__device__ __forceinline__ void wait_done(uint32_t* sync, int which, int n) {
  if (threadIdx.x == 0) {
    uint32_t* f = flag_of(sync, xcc_id(), which);
    const uint32_t want = done_mask(n);
    uint32_t spins = 0;
    while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != want) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > (1u << 24)) {  // never expected; guarantees the launch drains
        __hip_atomic_store(counter_of(sync, SYNC_ERR, 0), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

// Item `item` of `n` is finished: every wave's coherent stores are
// acknowledged before any counter moves.
__device__ __forceinline__ void signal_item(uint32_t* sync, int which, int item, int n) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int sub = item % kSubCounters;
    const uint32_t sub_target = (uint32_t)((n - sub + kSubCounters - 1) / kSubCounters);
    const uint32_t old =
        __hip_atomic_fetch_add(counter_of(sync, which, sub), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == sub_target - 1)
      for (int x = 0; x < kXcds; ++x)
        __hip_atomic_fetch_or(flag_of(sync, x, which), 1u << sub, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The workgroups of one role.  Block b runs on XCD b mod 8 as local slot
// j = b / 8, and slots j and j + nj/2 share a CU.  A role takes local slots on
// every XCD, so each stage's loads are spread over all eight L2s (whose miss
// tracking bounds a burst): the expert gate/up items take the second half
// of the slots (one per CU), router, shared gate/up and shared down items
// the start of the first half, and any further expert gate/up items the rest
// of it.  When the grid is not a whole number of XCD rounds every workgroup
// takes part, the role's items starting `shift` blocks in (so two roles do
// not start on the same blocks).
struct Role {
  int idx, count;  // this workgroup's index in the role (-1: not in it), role size
};
__device__ __forceinline__ Role role_slots(int b, int j0, int j1) {
  const int x = b % kXcds, j = b / kXcds;
  if (j < j0 || j >= j1) return Role{-1, (j1 - j0) * kXcds};
  return Role{(j - j0) * kXcds + x, (j1 - j0) * kXcds};
}
// slots [h, nj) first, then [f, h)
__device__ __forceinline__ Role role_two(int b, int f, int h, int nj) {
  const int x = b % kXcds, j = b / kXcds;
  const int count = (nj - f) * kXcds;
  if (j >= h) return Role{(j - h) * kXcds + x, count};
  if (j >= f) return Role{(nj - h + j - f) * kXcds + x, count};
  return Role{-1, count};
}
__device__ __forceinline__ Role role_all(int b, int nb, int shift) { return Role{(b + nb - shift % nb) % nb, nb}; }

// copy n halves (n multiple of 8) global -> LDS with 16-byte accesses
__device__ __forceinline__ void copy_halves(_Float16* dst, const void* src, int n) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(dst);
  for (int i = threadIdx.x; i < n / 8; i += blockDim.x) d[i] = s[i];
}

// dst[q] = src[index(q)] for q < n, 8 independent loads in flight per thread
// (a plain loop would wait for each load before issuing the next)
template <typename Dst, typename Index>
__device__ __forceinline__ void gather_batched(Dst* dst, const float* src, int n, Index index) {
  constexpr int B = 8;
  for (int base = 0; base < n; base += B * 256) {
    float v[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int q = base + u * 256 + (int)threadIdx.x;
      v[u] = q < n ? src[index(q)] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int q = base + u * 256 + (int)threadIdx.x;
      if (q < n) dst[q] = (Dst)v[u];
    }
  }
}

// h_e (n_up items of he_cols binary16 values, he_stride floats apart) ->
// act[ti][I], 16-byte loads, up to 8 in flight per thread (one round trip at
// real widths)
__device__ __forceinline__ void gather_h(_Float16* act, const float* h_e, const DecodePlan& p, int I) {
  constexpr int B = 8;
  const int cpi = p.he_cols / 8;  // 16-byte chunks per item
  const int n = p.n_up * cpi;
  for (int base = 0; base < n; base += B * 256) {
    uint4 v[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int c = base + u * 256 + (int)threadIdx.x;
      const int item = c / cpi;
      v[u] = c < n ? *reinterpret_cast<const uint4*>(h_e + (size_t)item * p.he_stride + 4 * (c % cpi))
                   : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int c = base + u * 256 + (int)threadIdx.x;
      const int item = c / cpi;
      const int ti = item / p.up_jblocks;
      const int j = (item % p.up_jblocks) * p.he_cols + 8 * (c % cpi);
      if (c < n && j < I) *reinterpret_cast<uint4*>(act + (size_t)ti * I + j) = v[u];
    }
  }
}

// per-lane 16-byte chunks of up to NB row-batches
template <int BITS, int NB, int MAXCPL>
struct Frag {
  uint4 q[NB][MAXCPL];
  float s[NB][MAXCPL];

  // rows[b]: this lane's row pointer in batch b (nullptr = masked); srow: its
  // scales (always a valid row).  Loads are unconditional: a masked lane reads
  // `safe` (a valid row) and zeroes the value, because a load under a branch
  // would be waited for inside the branch.
  __device__ __forceinline__ void load(const uint8_t* const rows[NB], const uint16_t* const srow[NB],
                                       const RowGeom& g, const uint8_t* safe) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int m = 0; m < MAXCPL; ++m) {
        const bool ok = rows[b] != nullptr && m < g.cpl;
        const int c = (lane % g.lpr) + g.lpr * (m < g.cpl ? m : 0);
        const uint4 t = *reinterpret_cast<const uint4*>((ok ? rows[b] : safe) + 16 * (size_t)c);
        const float sc = half_bits_to_float(srow[b][chunk_group<BITS>(c)]);
        q[b][m] = ok ? t : make_uint4(0, 0, 0, 0);
        s[b][m] = ok ? sc : 0.f;
      }
  }

  // acc[b][t] = this lane's share of row_b . act_t (same activations for every batch)
  template <int TT>
  __device__ __forceinline__ void dot_shared(const RowGeom& g, const _Float16* act, int stride, int T,
                                             float acc[NB][TT]) const {
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
#pragma unroll
              for (int b = 0; b < NB; ++b) acc[b][t] = fmaf(chunk_dot4(q[b][m], xp), s[b][m], acc[b][t]);
            } else {
              h2 xp[8];
              act16(a, xp);
#pragma unroll
              for (int b = 0; b < NB; ++b) acc[b][t] = fmaf(chunk_dot8(q[b][m], xp), s[b][m], acc[b][t]);
            }
          }
        }
      }
    }
  }

  // acc[b] = this lane's share of row_b . act_b (one activation vector per batch)
  __device__ __forceinline__ void dot_per_batch(const RowGeom& g, const _Float16* const act[NB], float acc[NB]) const {
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
            acc[b] = fmaf(chunk_dot4(q[b][m], xp), s[b][m], acc[b]);
          } else {
            h2 xp[8];
            act16(act[b] + EPC * c, xp);
            acc[b] = fmaf(chunk_dot8(q[b][m], xp), s[b][m], acc[b]);
          }
        }
      }
    }
  }
};

// ------------------------------------------------------------------ items

template <int MAXCPL>
__device__ void router_item(const DecodeArgs& a, int H, int item, const _Float16* xs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const RowGeom g = row_geom(H, 8);
  const int nrows = a.E + 1;
  const int rl = wave * g.rpb + lane / g.lpr;  // row within the item
  const int row = item * a.p.lg_rows + rl;
  const uint8_t* rows[1] = {row < nrows ? reinterpret_cast<const uint8_t*>(a.router_q) + (size_t)row * H : nullptr};
  const uint16_t* srow[1] = {a.router_s + (size_t)(row < nrows ? row : 0) * (H / kGroup)};
  Frag<8, 1, MAXCPL> f;
  f.load(rows, srow, g, reinterpret_cast<const uint8_t*>(a.router_q));
  float acc[1][kDecMaxT];
  f.template dot_shared<kDecMaxT>(g, xs, H, a.T, acc);
#pragma unroll
  for (int t = 0; t < kDecMaxT; ++t) {
    if (t < a.T) {
      const float v = lane_group_sum(acc[0][t], g.lpr);
      if (row < nrows && (lane % g.lpr) == 0) st_co(a.logits + ((size_t)item * a.T + t) * a.p.lg_stride + rl, v);
    }
  }
}

template <int MAXCPL>
__device__ void shup_item(const DecodeArgs& a, int H, int Is, int item, const _Float16* xs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const RowGeom g = row_geom(H, 8);
  const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sh13_q);
  const uint8_t* rows[4];
  const uint16_t* srow[4];
  int jl[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    jl[h] = (wave * 2 + h) * g.rpb + lane / g.lpr;
    const int j = item * a.p.hs_cols + jl[h];
    const bool ok = j < Is;
    rows[h] = ok ? base + (size_t)j * H : nullptr;
    rows[2 + h] = ok ? base + (size_t)(Is + j) * H : nullptr;
    srow[h] = a.sh13_s + (size_t)(ok ? j : 0) * (H / kGroup);
    srow[2 + h] = a.sh13_s + (size_t)(ok ? Is + j : 0) * (H / kGroup);
  }
  Frag<8, 4, MAXCPL> f;
  f.load(rows, srow, g, base);
  float acc[4][kDecMaxT];
  f.template dot_shared<kDecMaxT>(g, xs, H, a.T, acc);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int t = 0; t < kDecMaxT; ++t) {
      if (t < a.T) {
        const float gate = lane_group_sum(acc[h][t], g.lpr);
        const float up = lane_group_sum(acc[2 + h][t], g.lpr);
        if (item * a.p.hs_cols + jl[h] < Is && (lane % g.lpr) == 0)
          st_co(a.h_s + ((size_t)item * a.T + t) * a.p.hs_stride + jl[h], silu_f(gate) * up);
      }
    }
}

template <int MAXCPL>
__device__ void up_item(const DecodeArgs& a, int H, int I, int item, const _Float16* xs, const int (*ids)[kMaxTopK]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const RowGeom g = row_geom(H, 4);
  const int jblk = item % a.p.up_jblocks;
  const int ti = item / a.p.up_jblocks;
  const int t = ti / a.k, i = ti % a.k;
  const int e = ids[t][i];
  const size_t rb = (size_t)H / 2;
  const size_t ng = H / kGroup;
  const uint8_t* wbase = a.w13_q + (size_t)(e < 0 ? 0 : e) * 2 * I * rb;
  const uint16_t* sbase = a.w13_s + (size_t)(e < 0 ? 0 : e) * 2 * I * ng;
  const uint8_t* rows[8];
  const uint16_t* srow[8];
  int jl[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    jl[h] = (wave * 4 + h) * g.rpb + lane / g.lpr;
    const int j = jblk * a.p.he_cols + jl[h];
    const bool ok = e >= 0 && j < I;
    rows[h] = ok ? wbase + (size_t)j * rb : nullptr;
    rows[4 + h] = ok ? wbase + (size_t)(I + j) * rb : nullptr;
    srow[h] = sbase + (size_t)(ok ? j : 0) * ng;
    srow[4 + h] = sbase + (size_t)(ok ? I + j : 0) * ng;
  }
  Frag<4, 8, MAXCPL> f;
  f.load(rows, srow, g, wbase);
  float acc[8][1];
  f.template dot_shared<1>(g, xs + (size_t)t * H, H, 1, acc);
  uint16_t* dst = reinterpret_cast<uint16_t*>(a.h_e + (size_t)item * a.p.he_stride);  // binary16 values
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float gate = lane_group_sum(acc[h][0], g.lpr);
    const float up = lane_group_sum(acc[4 + h][0], g.lpr);
    if (jblk * a.p.he_cols + jl[h] < I && (lane % g.lpr) == 0) st_co_h(dst + jl[h], e >= 0 ? silu_f(gate) * up : 0.f);
  }
}

template <int MAXCPL>
__device__ void sd_item(const DecodeArgs& a, int H, int Is, int item, const _Float16* hs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const RowGeom g = row_geom(Is, 8);
  const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sh2_q);
  const size_t ng = Is / kGroup;
  const uint8_t* rows[4];
  const uint16_t* srow[4];
  int nl[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    nl[h] = (wave * 4 + h) * g.rpb + lane / g.lpr;
    const int n = item * a.p.ss_rows + nl[h];
    rows[h] = n < H ? base + (size_t)n * Is : nullptr;
    srow[h] = a.sh2_s + (size_t)(n < H ? n : 0) * ng;
  }
  Frag<8, 4, MAXCPL> f;
  f.load(rows, srow, g, base);
  float acc[4][kDecMaxT];
  f.template dot_shared<kDecMaxT>(g, hs, Is, a.T, acc);
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int t = 0; t < kDecMaxT; ++t) {
      if (t < a.T) {
        const float v = lane_group_sum(acc[h][t], g.lpr);
        if (item * a.p.ss_rows + nl[h] < H && (lane % g.lpr) == 0)
          st_co(a.s_sh + ((size_t)item * a.T + t) * a.p.ss_stride + nl[h], v);
      }
    }
}

// ------------------------------------------------------------------ kernel

// HC, IC, ISC: compile-time H, I, Is (0: taken from the arguments)
template <int MODE, int HC, int IC, int ISC>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  extern __shared__ uint4 smem_raw[];
  const int H = HC ? HC : a.H;
  const int I = IC ? IC : a.I;
  const int Is = ISC ? ISC : a.Is;
  constexpr int CPL8H = HC ? (HC / 1024 > 1 ? HC / 1024 : 1) : 4;
  constexpr int CPL4H = HC ? (HC / 2048 > 1 ? HC / 2048 : 1) : 2;
  constexpr int CPL8S = ISC ? (ISC / 1024 > 1 ? ISC / 1024 : 1) : 4;
  constexpr int CPL4I = IC ? (IC / 2048 > 1 ? IC / 2048 : 1) : 2;
  const DecodePlan& p = a.p;
  const int T = a.T, E = a.E, k = a.k;

  _Float16* act = reinterpret_cast<_Float16*>(smem_raw);  // x [T][H], later h_e [T][k][I]
  const int act_halves = max(T * H, T * k * I);
  _Float16* hs_lds = act + act_halves;                    // h_s [T][Is]
  __shared__ int s_ids[kDecMaxT][kMaxTopK];
  __shared__ float s_w[kDecMaxT][kMaxTopK];
  __shared__ float s_sig[kDecMaxT];
  __shared__ float s_red[4][64];
  __shared__ TopkScratch s_topk[kDecMaxT];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nb = gridDim.x, b = blockIdx.x;

  // DEC_BLOCK (the Chimera notebook, sections 7 and 10: post-attention
  // RMSNorm in front of the block, residual after it): the gain comes into
  // LDS with x, wave t sums token t's squares in a fixed order (so every
  // workgroup derives the same binary16 activations), and act is normalised in
  // place.
  __shared__ __attribute__((aligned(16))) _Float16 s_gain[MODE == DEC_BLOCK ? kMaxHidden : 8];
  __shared__ float s_rn[kDecMaxT];
  copy_halves(act, a.x, T * H);
  if (MODE == DEC_BLOCK) copy_halves(s_gain, a.gain, H);
  __syncthreads();
  if (MODE == DEC_BLOCK) {
    if (wave < T) {  // 8 halves (16 bytes) per lane and step
      const h8* row = reinterpret_cast<const h8*>(act + (size_t)wave * H);
      float ss = 0.f;
      for (int c = lane; c < H / 8; c += 64) {
        const h8 v = row[c];
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf((float)v[i], (float)v[i], ss);
      }
      ss = lane_group_sum(ss, 64);
      if (lane == 0) s_rn[wave] = 1.0f / sqrtf(ss / (float)H + a.eps);
    }
    __syncthreads();
    for (int q = tid; q < T * (H / 8); q += blockDim.x) {
      const int t = q / (H / 8), c = q - t * (H / 8);
      h8* p = reinterpret_cast<h8*>(act + (size_t)t * H) + c;
      const h8 gv = reinterpret_cast<const h8*>(s_gain)[c];
      h8 v = *p;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (_Float16)((float)v[i] * s_rn[t] * (float)gv[i]);
      *p = v;
    }
    __syncthreads();
  }

  // Roles by local slot (see role_slots); the down rows on every workgroup.
  const int nj = nb / kXcds, half = nj / 2;
  const int jr = (p.n_router + kXcds - 1) / kXcds, js = (p.n_shup + kXcds - 1) / kXcds;
  const int jd = MODE != DEC_EXPERTS ? (p.n_sd + kXcds - 1) / kXcds : 0;
  const bool split = nb % kXcds == 0 && nj % 2 == 0 && jr + js + jd < half;  // uniform
  const Role r_router = split ? role_slots(b, 0, jr) : role_all(b, nb, 0);
  const Role r_shup = split ? role_slots(b, jr, jr + js) : role_all(b, nb, p.n_router);
  const Role r_sd = split ? role_slots(b, jr + js, jr + js + jd) : role_all(b, nb, p.n_up);
  const Role r_up = split ? role_two(b, jr + js + jd, half, nj) : role_all(b, nb, 0);

  // ---------------- stage A
  if (MODE != DEC_EXPERTS) {
    if (r_router.idx >= 0)
      for (int item = r_router.idx; item < p.n_router; item += r_router.count) {
        router_item<CPL8H>(a, H, item, act);
        signal_item(a.sync, SYNC_ROUTER, item, p.n_router);
      }
    if (r_shup.idx >= 0)
      for (int item = r_shup.idx; item < p.n_shup; item += r_shup.count) {
        shup_item<CPL8H>(a, H, Is, item, act);
        signal_item(a.sync, SYNC_SHUP, item, p.n_shup);
      }
  }

  // ---------------- routing into LDS
  if (MODE != DEC_EXPERTS) {
    wait_done(a.sync, SYNC_ROUTER, p.n_router);
    // wave t ranks token t, reading its logits straight from the router
    // items' regions (lane l: experts 4l..4l+3, one 16-byte load)
    if (wave < T) {
      const int t = wave;
      const int e0 = 4 * lane;
      // both loads are issued before either value is used
      const float gate = a.logits[((size_t)(E / p.lg_rows) * T + t) * p.lg_stride + E % p.lg_rows];
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (e0 < p.n_router * p.lg_rows) {
        const float4 q = *reinterpret_cast<const float4*>(
            a.logits + ((size_t)(e0 / p.lg_rows) * T + t) * p.lg_stride + e0 % p.lg_rows);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
      }
      wave_topk(v, E, k, s_ids[t], s_w[t], s_topk[t]);
      if (lane == 0) s_sig[t] = sigmoid_f(gate);
    }
    __syncthreads();
    if (b == 0) {
      for (int q = tid; q < T * k; q += blockDim.x) {
        const int t = q / k, i = q % k;
        if (a.ids_out) a.ids_out[q] = s_ids[t][i];
        if (a.w_out) a.w_out[q] = s_w[t][i];
      }
      for (int t = tid; t < T; t += blockDim.x)
        if (a.sigma_out) a.sigma_out[t] = s_sig[t];
    }
  } else {
    for (int q = tid; q < T * k; q += blockDim.x) {
      const int t = q / k, i = q % k;
      const int e = a.ids_in[q];
      s_ids[t][i] = (e >= 0 && e < E) ? e : -1;  // invalid ids contribute nothing
      s_w[t][i] = a.w_in[q];
    }
    __syncthreads();
  }

  // ---------------- stage B
  if (r_up.idx >= 0)
    for (int item = r_up.idx; item < p.n_up; item += r_up.count) {
      up_item<CPL4H>(a, H, I, item, act, s_ids);
      signal_item(a.sync, SYNC_UP, item, p.n_up);
    }
  if (MODE != DEC_EXPERTS && r_sd.idx >= 0 && r_sd.idx < p.n_sd) {
    wait_done(a.sync, SYNC_SHUP, p.n_shup);
    gather_batched(hs_lds, a.h_s, T * Is, [&](int q) {
      const int t = q / Is, j = q % Is;
      return ((size_t)(j / p.hs_cols) * T + t) * p.hs_stride + j % p.hs_cols;
    });
    __syncthreads();
    for (int item = r_sd.idx; item < p.n_sd; item += r_sd.count) {
      sd_item<CPL8S>(a, H, Is, item, hs_lds);
      signal_item(a.sync, SYNC_SD, item, p.n_sd);
    }
  }

  // ---------------- stage C: down rows of every slot, combine, shared term
  {
    const RowGeom g = row_geom(I, 4);
    const int nblk = H / g.rpb;
    const size_t rb = (size_t)I / 2;
    const size_t ng = I / kGroup;
    bool h_ready = false;
    for (int item = b; item < p.n_down; item += nb) {
      const int t = item / nblk;
      const int n0 = (item % nblk) * g.rpb;
      const int n = n0 + lane / g.lpr;
      const uint8_t* rows[2];
      const uint16_t* srow[2];
      int slot[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int i = wave + 4 * q;
        const int e = i < k ? s_ids[t][i] : -1;
        slot[q] = e >= 0 ? i : -1;
        rows[q] = e >= 0 ? a.w2_q + ((size_t)e * H + n) * rb : nullptr;
        srow[q] = a.w2_s + ((size_t)(e >= 0 ? e : 0) * H + n) * ng;
      }
      Frag<4, 2, CPL4I> f;
      f.load(rows, srow, g, a.w2_q);
      // DEC_BLOCK: the residual of this item's outputs, loaded with the
      // weights (from a valid element for every thread: a load whose value is
      // selected at once would be waited for here)
      const uint16_t resid_bits = MODE == DEC_BLOCK ? a.x[(size_t)t * H + n0 + (tid < g.rpb ? tid : 0)] : 0;
      __builtin_amdgcn_sched_barrier(0);  // issue these loads before waiting
      if (!h_ready) {
        wait_done(a.sync, SYNC_UP, p.n_up);
        if (MODE != DEC_EXPERTS) wait_done(a.sync, SYNC_SD, p.n_sd);
        gather_h(act, a.h_e, p, I);
        __syncthreads();
        h_ready = true;
      }
      const _Float16* hact[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) hact[q] = slot[q] >= 0 ? act + ((size_t)t * k + slot[q]) * I : nullptr;
      float acc[2];
      f.dot_per_batch(g, hact, acc);
      float part = 0.f;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float y = lane_group_sum(acc[q], g.lpr);
        if (slot[q] >= 0) part += s_w[t][slot[q]] * y;
      }
      if ((lane % g.lpr) == 0) s_red[wave][lane / g.lpr] = part;
      __syncthreads();
      if (tid < g.rpb) {
        float v = s_red[0][tid] + s_red[1][tid] + s_red[2][tid] + s_red[3][tid];
        const int nn = n0 + tid;
        if (MODE != DEC_EXPERTS)
          v += s_sig[t] * a.s_sh[((size_t)(nn / p.ss_rows) * T + t) * p.ss_stride + nn % p.ss_rows];
        if (MODE == DEC_BLOCK) v += half_bits_to_float(resid_bits);
        const _Float16 hv = (_Float16)v;
        a.out[(size_t)t * H + nn] = __builtin_bit_cast(uint16_t, hv);
      }
      __syncthreads();
    }
  }

  // ---------------- drain: the last workgroup out clears the counters
  // (exits count on sub-counters too: 512 increments of one counter would
  // serialise at the memory for microseconds)
  __shared__ int s_last;
  __syncthreads();
  if (tid == 0) {
    const int sub = b % kSubCounters;
    const uint32_t sub_target = (uint32_t)((nb - sub + kSubCounters - 1) / kSubCounters);
    bool last = false;
    if (__hip_atomic_fetch_add(counter_of(a.sync, SYNC_EXIT, sub), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        sub_target - 1) {
      const uint32_t top_target = (uint32_t)(nb < kSubCounters ? nb : kSubCounters);
      last = __hip_atomic_fetch_add(counter_of(a.sync, SYNC_EXIT, kSubCounters), 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == top_target - 1;
    }
    s_last = last;
  }
  __syncthreads();
  if (s_last) {  // one store per thread: counters, then flags
    constexpr int NC = (SYNC_EXIT + 1) * (kSubCounters + 1), NF = (SYNC_EXIT + 1) * kXcds;
    for (int q = tid; q < NC + NF; q += blockDim.x) {
      uint32_t* w = q < NC ? counter_of(a.sync, q / (kSubCounters + 1), q % (kSubCounters + 1))
                           : flag_of(a.sync, (q - NC) % kXcds, (q - NC) / kXcds);
      __hip_atomic_store(w, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------------ host side

bool decode_real_widths(int H, int I, int Is) { return H == 2048 && I == 512 && Is == 512; }

template <int MODE>
static int occupancy(bool real, size_t lds) {
  int n = 0;
  hipError_t err = real ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<MODE, 2048, 512, 512>, 256, lds)
                        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<MODE, 0, 0, 0>, 256, lds);
  return err == hipSuccess ? n : 0;
}

int decode_blocks_per_cu(int mode, bool real, size_t lds_bytes) {
  if (mode == DEC_BLOCK) return occupancy<DEC_BLOCK>(real, lds_bytes);
  return mode == DEC_FORWARD ? occupancy<DEC_FORWARD>(real, lds_bytes) : occupancy<DEC_EXPERTS>(real, lds_bytes);
}

int launch_decode(const DecodeArgs& a, int mode, int grid, size_t lds_bytes, hipStream_t s) {
  const bool real = decode_real_widths(a.H, a.I, a.Is);
  if (mode == DEC_FORWARD) {
    if (real) hipLaunchKernelGGL((decode_kernel<DEC_FORWARD, 2048, 512, 512>), dim3(grid), dim3(256), lds_bytes, s, a);
    else hipLaunchKernelGGL((decode_kernel<DEC_FORWARD, 0, 0, 0>), dim3(grid), dim3(256), lds_bytes, s, a);
  } else if (mode == DEC_BLOCK) {
    if (real) hipLaunchKernelGGL((decode_kernel<DEC_BLOCK, 2048, 512, 512>), dim3(grid), dim3(256), lds_bytes, s, a);
    else hipLaunchKernelGGL((decode_kernel<DEC_BLOCK, 0, 0, 0>), dim3(grid), dim3(256), lds_bytes, s, a);
  } else {
    if (real) hipLaunchKernelGGL((decode_kernel<DEC_EXPERTS, 2048, 512, 512>), dim3(grid), dim3(256), lds_bytes, s, a);
    else hipLaunchKernelGGL((decode_kernel<DEC_EXPERTS, 0, 0, 0>), dim3(grid), dim3(256), lds_bytes, s, a);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace moe
