// Few-token path of the routed MoE block: one persistent launch.
//
// The block (the Chimera notebook, section 5): out = routed + sigmoid(x . W_sg)
// * shared, where the routed part is the renormalised top-k mixture of int4
// SwiGLU experts (section 5.2 ordering: softmax -> top-k -> renormalise) and
// the router rows are int8 group-64 rows stacked with the shared-gate row (the
// TensorFold PR, "Design").
//
// Work is split into items executed by a grid of co-resident workgroups.  Items
// hand results to each other through agent-scope counters instead of kernel
// boundaries (one launch costs about as much as the whole layer's HBM time at
// one token):
//   A  router rows (logits) | shared-expert gate/up rows (h_s)
//   B  expert gate/up rows of the k selected experts (h_e)   <- router
//      shared-expert down rows (s)                           <- shared gate/up
//   C  expert down rows + weighted combine + sigma * s       <- B
// Every workgroup recomputes the top-k from the logits itself (one wave per
// token), so no extra hand-off is needed between routing and the experts.
// The weights of a workgroup's first C item are loaded before it waits.
//
// Hand-off without cache maintenance: on gfx950 each XCD has its own L2, and
// agent-scope acquire/release fences invalidate / write back a whole L2.  The
// values passed between workgroups (logits, h, s) are therefore written and
// read with device-coherent (agent-scope) relaxed atomic accesses, which do
// not leave stale or dirty copies in an XCD's L2.  A producer waits until its
// stores are acknowledged (vmcnt 0) before it bumps the counter; a consumer
// polls the counter and then reads the values with the same coherent loads.
#include "decode.hpp"
#include "gemv.hpp"

namespace moe {

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ void st_co(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_co(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wait_count(uint32_t* sync, int which, uint32_t target) {
  if (threadIdx.x == 0) {
    uint32_t* ctr = sync + which * kSyncStride;
    uint32_t spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > (1u << 24)) {  // never expected; guarantees the launch drains
        __hip_atomic_store(sync + SYNC_ERR * kSyncStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

// every wave's coherent stores are acknowledged before the counter moves
__device__ __forceinline__ void signal_item(uint32_t* sync, int which) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(sync + which * kSyncStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// n coherent floats (n even, src 8-byte aligned) -> LDS halves.  Loads are
// issued in batches of 8 per thread before any is used, so a copy costs one
// memory round trip per batch rather than one per element.
__device__ __forceinline__ void copy_co_to_halves(_Float16* dst, const float* src, int n) {
  const uint64_t* s2 = reinterpret_cast<const uint64_t*>(src);
  const int n2 = n / 2;
  constexpr int B = 8;
  for (int base = 0; base < n2; base += B * 256) {
    uint64_t v[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int i = base + u * 256 + (int)threadIdx.x;
      v[u] = i < n2 ? __hip_atomic_load(const_cast<uint64_t*>(s2 + i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                    : 0ull;
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int i = base + u * 256 + (int)threadIdx.x;
      if (i < n2) {
        h2 hv;
        hv[0] = (_Float16)__builtin_bit_cast(float, (uint32_t)v[u]);
        hv[1] = (_Float16)__builtin_bit_cast(float, (uint32_t)(v[u] >> 32));
        reinterpret_cast<h2*>(dst)[i] = hv;
      }
    }
  }
}

// n coherent floats -> LDS floats, batched the same way
__device__ __forceinline__ void copy_co_floats(float* dst, const float* src, int n) {
  constexpr int B = 8;
  for (int base = 0; base < n; base += B * 256) {
    float v[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int i = base + u * 256 + (int)threadIdx.x;
      v[u] = i < n ? ld_co(src + i) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int i = base + u * 256 + (int)threadIdx.x;
      if (i < n) dst[i] = v[u];
    }
  }
}

// copy n halves (n multiple of 8) global -> LDS with 16-byte accesses
__device__ __forceinline__ void copy_halves(_Float16* dst, const void* src, int n) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(dst);
  for (int i = threadIdx.x; i < n / 8; i += blockDim.x) d[i] = s[i];
}

// per-lane 16-byte chunks of up to NB row-batches
template <int BITS, int NB, int MAXCPL>
struct Frag {
  uint4 q[NB][MAXCPL];
  float s[NB][MAXCPL];

  // rows[b]: this lane's row pointer in batch b (nullptr = masked); srow: its scales
  __device__ __forceinline__ void load(const uint8_t* const rows[NB], const uint16_t* const srow[NB],
                                       const RowGeom& g) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int m = 0; m < MAXCPL; ++m) {
        q[b][m] = make_uint4(0, 0, 0, 0);
        s[b][m] = 0.f;
        if (rows[b] != nullptr && m < g.cpl) {
          const int c = (lane % g.lpr) + g.lpr * m;
          q[b][m] = *reinterpret_cast<const uint4*>(rows[b] + 16 * (size_t)c);
          s[b][m] = half_bits_to_float(srow[b][chunk_group<BITS>(c)]);
        }
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

// A: router rows (and the stacked shared-gate row) -> logits[t][row]
__device__ void router_item(const DecodeArgs& a, int item, const _Float16* xs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const RowGeom g = row_geom(a.H, 8);
  const int nrows = a.E + 1;
  const int row = (item * 4 + wave) * g.rpb + lane / g.lpr;
  const size_t rb = (size_t)a.H;
  const uint8_t* rows[1] = {row < nrows ? reinterpret_cast<const uint8_t*>(a.router_q) + row * rb : nullptr};
  const uint16_t* srow[1] = {a.router_s + (size_t)(row < nrows ? row : 0) * (a.H / kGroup)};
  Frag<8, 1, 4> f;
  f.load(rows, srow, g);
  float acc[1][kDecMaxT];
  f.dot_shared<kDecMaxT>(g, xs, a.H, a.T, acc);
#pragma unroll
  for (int t = 0; t < kDecMaxT; ++t) {
    const float v = group_sum(acc[0][t], g.lpr);
    if (t < a.T && row < nrows && (lane % g.lpr) == 0) st_co(a.logits + (size_t)t * nrows + row, v);
  }
}

// A: shared expert gate/up rows -> h_s[t][j] = silu(gate) * up
__device__ void shup_item(const DecodeArgs& a, int item, const _Float16* xs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const RowGeom g = row_geom(a.H, 8);
  const int jw = 2 * g.rpb;  // j per wave
  const int j0 = (item * 4 + wave) * jw;
  const size_t rb = (size_t)a.H;
  const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sh13_q);
  const uint8_t* rows[4];
  const uint16_t* srow[4];
  int jj[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = j0 + h * g.rpb + lane / g.lpr;
    jj[h] = j;
    const bool ok = j < a.Is;
    rows[h] = ok ? base + (size_t)j * rb : nullptr;
    rows[2 + h] = ok ? base + (size_t)(a.Is + j) * rb : nullptr;
    srow[h] = a.sh13_s + (size_t)(ok ? j : 0) * (a.H / kGroup);
    srow[2 + h] = a.sh13_s + (size_t)(ok ? a.Is + j : 0) * (a.H / kGroup);
  }
  Frag<8, 4, 4> f;
  f.load(rows, srow, g);
  float acc[4][kDecMaxT];
  f.dot_shared<kDecMaxT>(g, xs, a.H, a.T, acc);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int t = 0; t < kDecMaxT; ++t) {
      const float gate = group_sum(acc[h][t], g.lpr);
      const float up = group_sum(acc[2 + h][t], g.lpr);
      if (t < a.T && jj[h] < a.Is && (lane % g.lpr) == 0)
        st_co(a.h_s + (size_t)t * a.Is + jj[h], silu_f(gate) * up);
    }
}

// B: one (token, slot, j-block): expert gate/up rows -> h_e[t][i][j]
__device__ void up_item(const DecodeArgs& a, int item, const _Float16* xs, const int (*ids)[kMaxTopK]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const RowGeom g = row_geom(a.H, 4);
  const int jblk = item % a.up_jblocks;
  const int ti = item / a.up_jblocks;
  const int t = ti / a.k, i = ti % a.k;
  const int e = ids[t][i];
  const int jw = 4 * g.rpb;
  const int j0 = (jblk * 4 + wave) * jw;
  const size_t rb = (size_t)a.H / 2;
  const size_t ng = a.H / kGroup;
  const uint8_t* wbase = a.w13_q + (size_t)(e < 0 ? 0 : e) * 2 * a.I * rb;
  const uint16_t* sbase = a.w13_s + (size_t)(e < 0 ? 0 : e) * 2 * a.I * ng;
  const uint8_t* rows[8];
  const uint16_t* srow[8];
  int jj[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int j = j0 + h * g.rpb + lane / g.lpr;
    jj[h] = j;
    const bool ok = e >= 0 && j < a.I;
    rows[h] = ok ? wbase + (size_t)j * rb : nullptr;
    rows[4 + h] = ok ? wbase + (size_t)(a.I + j) * rb : nullptr;
    srow[h] = sbase + (size_t)(ok ? j : 0) * ng;
    srow[4 + h] = sbase + (size_t)(ok ? a.I + j : 0) * ng;
  }
  Frag<4, 8, 2> f;
  f.load(rows, srow, g);
  float acc[8][1];
  f.dot_shared<1>(g, xs + (size_t)t * a.H, a.H, 1, acc);
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float gate = group_sum(acc[h][0], g.lpr);
    const float up = group_sum(acc[4 + h][0], g.lpr);
    if (jj[h] < a.I && (lane % g.lpr) == 0)
      st_co(a.h_e + ((size_t)t * a.k + i) * a.I + jj[h], e >= 0 ? silu_f(gate) * up : 0.f);
  }
}

// B: shared expert down rows -> s_sh[t][n]
__device__ void sd_item(const DecodeArgs& a, int item, const _Float16* hs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const RowGeom g = row_geom(a.Is, 8);
  const int rw = 4 * g.rpb;
  const int n0 = (item * 4 + wave) * rw;
  const size_t rb = (size_t)a.Is;
  const size_t ng = a.Is / kGroup;
  const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sh2_q);
  const uint8_t* rows[4];
  const uint16_t* srow[4];
  int nn[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int n = n0 + h * g.rpb + lane / g.lpr;
    nn[h] = n;
    rows[h] = n < a.H ? base + (size_t)n * rb : nullptr;
    srow[h] = a.sh2_s + (size_t)(n < a.H ? n : 0) * ng;
  }
  Frag<8, 4, 4> f;
  f.load(rows, srow, g);
  float acc[4][kDecMaxT];
  f.dot_shared<kDecMaxT>(g, hs, a.Is, a.T, acc);
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int t = 0; t < kDecMaxT; ++t) {
      const float v = group_sum(acc[h][t], g.lpr);
      if (t < a.T && nn[h] < a.H && (lane % g.lpr) == 0) st_co(a.s_sh + (size_t)t * a.H + nn[h], v);
    }
}

// ------------------------------------------------------------------ kernel

template <int MODE>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  extern __shared__ uint4 smem_raw[];
  _Float16* act = reinterpret_cast<_Float16*>(smem_raw);  // x [T][H], later h_e [T][k][I]
  const int act_halves = max(a.T * a.H, a.T * a.k * a.I);
  _Float16* hs_lds = act + act_halves;                    // h_s [T][Is]
  __shared__ int s_ids[kDecMaxT][kMaxTopK];
  __shared__ float s_w[kDecMaxT][kMaxTopK];
  __shared__ float s_sig[kDecMaxT];
  __shared__ float s_red[4][64];
  __shared__ float s_logits_raw[kDecMaxT * (kMaxExperts + 1)];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nb = gridDim.x, b = blockIdx.x;
  const int T = a.T;

  copy_halves(act, a.x, T * a.H);
  __syncthreads();

  // ---------------- stage A
  if (MODE == DEC_FORWARD) {
    const int nA = a.n_router + a.n_shup;
    for (int item = b; item < nA; item += nb) {
      const bool is_router = item < a.n_router;
      if (is_router) router_item(a, item, act);
      else shup_item(a, item - a.n_router, act);
      signal_item(a.sync, is_router ? SYNC_ROUTER : SYNC_SHUP);
    }
  }

  // ---------------- routing into LDS
  if (MODE == DEC_FORWARD) {
    wait_count(a.sync, SYNC_ROUTER, a.n_router);
    const int nrows = a.E + 1;
    copy_co_floats(s_logits_raw, a.logits, T * nrows);  // [T][E+1]
    __syncthreads();
    for (int t = wave; t < T; t += 4) {
      wave_topk(s_logits_raw + t * nrows, a.E, a.k, s_ids[t], s_w[t]);
      if (lane == 0) s_sig[t] = sigmoid_f(s_logits_raw[t * nrows + a.E]);
    }
    __syncthreads();
    if (b == 0) {
      for (int p = tid; p < T * a.k; p += blockDim.x) {
        const int t = p / a.k, i = p % a.k;
        if (a.ids_out) a.ids_out[p] = s_ids[t][i];
        if (a.w_out) a.w_out[p] = s_w[t][i];
      }
      for (int t = tid; t < T; t += blockDim.x)
        if (a.sigma_out) a.sigma_out[t] = s_sig[t];
      if (a.logits_out)
        for (int p = tid; p < T * nrows; p += blockDim.x) a.logits_out[p] = s_logits_raw[p];
    }
  } else {
    for (int p = tid; p < T * a.k; p += blockDim.x) {
      const int t = p / a.k, i = p % a.k;
      const int e = a.ids_in[p];
      s_ids[t][i] = (e >= 0 && e < a.E) ? e : -1;  // invalid ids contribute nothing
      s_w[t][i] = a.w_in[p];
    }
    __syncthreads();
  }

  // ---------------- stage B
  {
    const int nB = a.n_up + (MODE == DEC_FORWARD ? a.n_sd : 0);
    bool hs_ready = false;
    for (int item = b; item < nB; item += nb) {
      if (item < a.n_up) {
        up_item(a, item, act, s_ids);
        signal_item(a.sync, SYNC_UP);
      } else {
        if (!hs_ready) {
          wait_count(a.sync, SYNC_SHUP, a.n_shup);
          copy_co_to_halves(hs_lds, a.h_s, T * a.Is);
          __syncthreads();
          hs_ready = true;
        }
        sd_item(a, item - a.n_up, hs_lds);
        signal_item(a.sync, SYNC_SD);
      }
    }
  }

  // ---------------- stage C: down rows of every slot, combine, shared term
  {
    const RowGeom g = row_geom(a.I, 4);
    const int nblk = a.H / g.rpb;
    const size_t rb = (size_t)a.I / 2;
    const size_t ng = a.I / kGroup;
    bool h_ready = false;
    for (int item = b; item < a.n_down; item += nb) {
      const int t = item / nblk;
      const int n0 = (item % nblk) * g.rpb;
      const int n = n0 + lane / g.lpr;
      const uint8_t* rows[2];
      const uint16_t* srow[2];
      int slot[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int i = wave + 4 * q;
        const int e = i < a.k ? s_ids[t][i] : -1;
        slot[q] = e >= 0 ? i : -1;
        rows[q] = e >= 0 ? a.w2_q + ((size_t)e * a.H + n) * rb : nullptr;
        srow[q] = a.w2_s + ((size_t)(e >= 0 ? e : 0) * a.H + n) * ng;
      }
      Frag<4, 2, 2> f;
      f.load(rows, srow, g);
      if (!h_ready) {
        wait_count(a.sync, SYNC_UP, a.n_up);
        if (MODE == DEC_FORWARD) wait_count(a.sync, SYNC_SD, a.n_sd);
        copy_co_to_halves(act, a.h_e, T * a.k * a.I);
        __syncthreads();
        h_ready = true;
      }
      const _Float16* hact[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) hact[q] = slot[q] >= 0 ? act + ((size_t)t * a.k + slot[q]) * a.I : nullptr;
      float acc[2];
      f.dot_per_batch(g, hact, acc);
      float part = 0.f;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float y = group_sum(acc[q], g.lpr);
        if (slot[q] >= 0) part += s_w[t][slot[q]] * y;
      }
      if ((lane % g.lpr) == 0) s_red[wave][lane / g.lpr] = part;
      __syncthreads();
      if (tid < g.rpb) {
        float v = s_red[0][tid] + s_red[1][tid] + s_red[2][tid] + s_red[3][tid];
        const int nn = n0 + tid;
        if (MODE == DEC_FORWARD) v += s_sig[t] * ld_co(a.s_sh + (size_t)t * a.H + nn);
        const _Float16 hv = (_Float16)v;
        a.out[(size_t)t * a.H + nn] = __builtin_bit_cast(uint16_t, hv);
      }
      __syncthreads();
    }
  }

  // ---------------- drain: the last workgroup out clears the counters
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.sync + SYNC_EXIT * kSyncStride, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    if (old == (uint32_t)nb - 1) {
      for (int w = 0; w < SYNC_EXIT + 1; ++w)
        __hip_atomic_store(a.sync + w * kSyncStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------------ host side

int decode_blocks_per_cu(int mode, size_t lds_bytes) {
  int n = 0;
  hipError_t err = mode == DEC_FORWARD
                       ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<DEC_FORWARD>, 256, lds_bytes)
                       : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<DEC_EXPERTS>, 256, lds_bytes);
  return err == hipSuccess ? n : 0;
}

int launch_decode(const DecodeArgs& a, int mode, int grid, size_t lds_bytes, hipStream_t s) {
  if (mode == DEC_FORWARD)
    hipLaunchKernelGGL(decode_kernel<DEC_FORWARD>, dim3(grid), dim3(256), lds_bytes, s, a);
  else
    hipLaunchKernelGGL(decode_kernel<DEC_EXPERTS>, dim3(grid), dim3(256), lds_bytes, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace moe
