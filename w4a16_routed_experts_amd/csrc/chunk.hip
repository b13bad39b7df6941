// Multi-token path of the routed MoE block: grouped GEMMs on MFMA.
//
// The same block as the decode path (the Chimera notebook, section 5; the
// router ordering of section 5.2; int8 group-64 router rows stacked with the
// shared gate, the TensorFold PR "Design"), organised for many tokens:
//   1. router GEMM          logits[T][E+1]               (int8 rows, MFMA)
//   2. top-k per token      ids, renormalised weights, sigma
//   3. bucketing            (token, slot) pairs sorted by expert, then pair
//                           index; 32-row tiles per expert; shared-expert tiles
//   4. gate/up GEMM         h[row][I] = silu(x W_gate^T) * (x W_up^T)  (fp16)
//   5. down GEMM            y[row][H] = w * (h W_down^T)                (fp32)
//   6. combine              out[t] = sum_i y[pos(t,i)] + sigma_t * s[t]
// Each expert's weights are streamed once per 32-row tile; a tile's rows are
// the tokens routed to that expert.  Scales are applied per 64-wide K group
// to fp32 partial sums, so the MFMA products of binary16 codes and binary16
// activations are exact.
#include "chunk.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// MFMA tile core: acc[f] += A[32][K] . W_f[32][K]^T for NF fragments of 32
// weight rows.  MFMA 32x32x16 f16: lane l works on weight row (l % 32) of a
// fragment and K offsets 32*(l/32) .. +32 of each 64-wide group, so the 16
// codes of every MFMA step share one scale.
// ---------------------------------------------------------------------------

static constexpr int kBM = 32;                 // tile rows (tokens)
static constexpr int kKB = 256;                // K per LDS stage
static constexpr int kLdsStride = kKB + 8;     // halves per LDS row (padding)

// Stage A[32][kb .. kb+kKB) into LDS, each 8-element run permuted to the
// (0,4,1,5,2,6,3,7) order of the weight conversion.
__device__ __forceinline__ void stage_a(_Float16* lds, const _Float16* const* rows, int kb, int K) {
  const int nchunk = kKB / 8;  // 16-byte chunks per row
  for (int idx = threadIdx.x; idx < kBM * nchunk; idx += blockDim.x) {
    const int m = idx / nchunk, c = idx % nchunk;
    const int k = kb + 8 * c;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (rows[m] != nullptr && k < K) v = *reinterpret_cast<const uint4*>(rows[m] + k);
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
    perm8_words(x, o);
    *reinterpret_cast<uint4*>(lds + m * kLdsStride + 8 * c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Weight codes of this lane for one 64-group: K offsets kg + 32*(lane/32) .. +32
template <int BITS>
struct BChunk {
  uint4 q[BITS == 4 ? 1 : 2];
};

template <int BITS>
__device__ __forceinline__ BChunk<BITS> load_b(const uint8_t* row, int kg) {
  const int g = (threadIdx.x & 63) >> 5;
  BChunk<BITS> c;
  if (row == nullptr) {
#pragma unroll
    for (int i = 0; i < (BITS == 4 ? 1 : 2); ++i) c.q[i] = make_uint4(0, 0, 0, 0);
    return c;
  }
  if (BITS == 4) {
    c.q[0] = *reinterpret_cast<const uint4*>(row + (kg + 32 * g) / 2);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(row + kg + 32 * g);
    c.q[0] = p[0];
    c.q[1] = p[1];
  }
  return c;
}

// operand of MFMA step s (0..3) from a loaded chunk
template <int BITS>
__device__ __forceinline__ h8 b_step(const BChunk<BITS>& c, int s) {
  h2 w[4];
  if (BITS == 4) {
    const uint32_t ws[4] = {c.q[0].x, c.q[0].y, c.q[0].z, c.q[0].w};
    int4x8_to_h2x4(ws[s], w);
  } else {
    const uint32_t ws[8] = {c.q[0].x, c.q[0].y, c.q[0].z, c.q[0].w, c.q[1].x, c.q[1].y, c.q[1].z, c.q[1].w};
    int8x8_to_h2x4(ws[2 * s], ws[2 * s + 1], w);
  }
  h8 r;
  r[0] = w[0][0]; r[1] = w[0][1]; r[2] = w[1][0]; r[3] = w[1][1];
  r[4] = w[2][0]; r[5] = w[2][1]; r[6] = w[3][0]; r[7] = w[3][1];
  return r;
}

// acc[f] += A . W_f^T over K (a multiple of 64).  brow[f]: this lane's weight
// row (nullptr = zero row); bscale[f]: its scales.
template <int BITS, int NF>
__device__ __forceinline__ void tile_gemm(_Float16* lds, const _Float16* const* arows, int K,
                                          const uint8_t* const brow[NF], const uint16_t* const bscale[NF],
                                          f16v acc[NF]) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 31, g = lane >> 5;
  for (int kb = 0; kb < K; kb += kKB) {
    __syncthreads();
    stage_a(lds, arows, kb, K);
    __syncthreads();
    const int ngr = min(kKB, K - kb) / kGroup;
    for (int gi = 0; gi < ngr; ++gi) {
      const int kg = kb + gi * kGroup;
      BChunk<BITS> bc[NF];
      float sc[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        bc[f] = load_b<BITS>(brow[f], kg);
        sc[f] = brow[f] ? half_bits_to_float(bscale[f][kg / kGroup]) : 0.f;
      }
      const _Float16* ap = lds + m * kLdsStride + gi * kGroup + 32 * g;
      h8 av[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) av[s] = *reinterpret_cast<const h8*>(ap + 8 * s);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        f16v p = {};
#pragma unroll
        for (int s = 0; s < 4; ++s) p = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[s], b_step<BITS>(bc[f], s), p, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[f][i] = fmaf(p[i], sc[f], acc[f][i]);
      }
    }
  }
}

// row of the 32x32 accumulator held in element i of this lane
__device__ __forceinline__ int acc_row(int i) { return 8 * (i >> 2) + 4 * ((threadIdx.x & 63) >> 5) + (i & 3); }

// ---------------------------------------------------------------------------
// 1. router GEMM: logits[t][r], r < E+1
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_gemm_kernel(ChunkArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[kBM * kLdsStride];
  __shared__ const _Float16* arows[kBM];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * kBM;
  const int nrows = a.E + 1;
  if (threadIdx.x < kBM) {
    const int t = t0 + threadIdx.x;
    arows[threadIdx.x] = t < a.T ? reinterpret_cast<const _Float16*>(a.x) + (size_t)t * a.H : nullptr;
  }
  const int r = blockIdx.y * 128 + wave * 32 + (lane & 31);
  const uint8_t* brow[1] = {r < nrows ? reinterpret_cast<const uint8_t*>(a.router_q) + (size_t)r * a.H : nullptr};
  const uint16_t* bsc[1] = {a.router_s + (size_t)(r < nrows ? r : 0) * (a.H / kGroup)};
  f16v acc[1] = {};
  tile_gemm<8, 1>(lds, arows, a.H, brow, bsc, acc);
  if (r < nrows) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = t0 + acc_row(i);
      if (t < a.T) a.logits[(size_t)t * nrows + r] = acc[0][i];
    }
  }
}

// ---------------------------------------------------------------------------
// 2. top-k per token (one wave per token)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void topk_kernel(ChunkArgs a) {
  __shared__ int s_ids[4][kMaxTopK];
  __shared__ float s_w[4][kMaxTopK];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.T) return;
  const int nrows = a.E + 1;
  wave_topk(a.logits + (size_t)t * nrows, a.E, a.k, s_ids[wave], s_w[wave]);
  if (lane < a.k) {
    a.ids[(size_t)t * a.k + lane] = s_ids[wave][lane];
    a.wts[(size_t)t * a.k + lane] = s_w[wave][lane];
  }
  if (lane == 0) a.sigma[t] = sigmoid_f(a.logits[(size_t)t * nrows + a.E]);
}

// ---------------------------------------------------------------------------
// 3. bucketing: one workgroup of 1024 threads (16 waves)
//
// Pairs p = t*k + i are ordered by (expert, p): a stable counting sort.  Each
// wave owns a contiguous run of pairs; ranks inside a 64-pair batch come from
// ballots over the 8 bits of the expert id.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t peers_of(int e) {
  uint64_t peers = ~0ull;
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const uint64_t m = __ballot((e >> bit) & 1);
    peers &= ((e >> bit) & 1) ? m : ~m;
  }
  return peers;
}

__global__ __launch_bounds__(1024) void bucket_kernel(ChunkArgs a) {
  __shared__ int hist[16][kMaxExperts + 1];  // per-wave counts, then per-wave bases
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_tiles[kMaxExperts + 1];
  __shared__ int s_total;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int P = a.T * a.k;
  const int E = a.E;
  const int per = (P + 15) / 16;
  const int p_begin = min(P, wave * per), p_end = min(P, p_begin + per);
  const uint64_t lt = (1ull << lane) - 1ull;

  for (int i = threadIdx.x; i < 16 * (kMaxExperts + 1); i += blockDim.x) (&hist[0][0])[i] = 0;
  __syncthreads();
  // per-wave histograms (ids outside [0, E) are dropped: they never index weights)
  for (int p0 = p_begin; p0 < p_end; p0 += 64) {
    const int p = p0 + lane;
    const int e = p < p_end ? a.ids[p] : -1;
    const bool ok = e >= 0 && e < E;
    const uint64_t pe = peers_of(ok ? e : 255) & __ballot(ok);
    if (ok && (pe & lt) == 0) hist[wave][e] += __popcll(pe);  // one leader per expert
  }
  __syncthreads();
  // exclusive scan over experts of the totals; per-wave bases
  if (threadIdx.x < kMaxExperts + 1) {
    const int e = threadIdx.x;
    int tot = 0;
    if (e < E)
      for (int w = 0; w < 16; ++w) { const int c = hist[w][e]; hist[w][e] = tot; tot += c; }
    s_off[e] = e < E ? tot : 0;  // counts for now
    s_tiles[e] = e < E ? (tot + kBM - 1) / kBM : 0;
  }
  __syncthreads();
  if (wave == 0) {  // scans of counts and tile counts (E <= 256: 4 per lane)
    int c[4], tl[4];
    int sc = 0, st = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      c[j] = e < E ? s_off[e] : 0;
      tl[j] = e < E ? s_tiles[e] : 0;
      sc += c[j];
      st += tl[j];
    }
    int ic = sc, it = st;
    for (int d = 1; d < 64; d <<= 1) {
      const int uc = __shfl_up(ic, d, 64), ut = __shfl_up(it, d, 64);
      if (lane >= d) { ic += uc; it += ut; }
    }
    int ec = ic - sc, et = it - st;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      if (e <= kMaxExperts) { s_off[e] = ec; s_tiles[e] = et; }
      ec += c[j];
      et += tl[j];
    }
    if (lane == 63) {
      s_total = ic;  // valid pairs
      a.offsets[E] = ic;
      *a.n_tiles = it;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) a.offsets[e] = s_off[e];
  {
    const int total = s_total;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      const int start = s_off[e];
      const int end = (e + 1 < E) ? s_off[e + 1] : total;
      int ti = s_tiles[e];
      for (int r = start; r < end; r += kBM, ++ti) a.tiles[ti] = make_int4(e, r, min(kBM, end - r), 0);
    }
  }
  // stable scatter: position of pair p in expert-major order
  for (int p0 = p_begin; p0 < p_end; p0 += 64) {
    const int p = p0 + lane;
    const int e = p < p_end ? a.ids[p] : -1;
    const bool ok = e >= 0 && e < E;
    const uint64_t pe = peers_of(ok ? e : 255) & __ballot(ok);
    if (ok) {
      const int pos = s_off[e] + hist[wave][e] + __popcll(pe & lt);
      a.sorted_pair[pos] = p;
      a.pos_of_pair[p] = pos;
    } else if (p < p_end) {
      a.pos_of_pair[p] = -1;
    }
    if (ok && (pe & lt) == 0) hist[wave][e] += __popcll(pe);
  }
}

// ---------------------------------------------------------------------------
// 4. gate/up GEMM with SwiGLU epilogue.  blockIdx.x: tile (routed tiles, then
// shared-expert tiles); blockIdx.y: block of 128 intermediate columns.
// ---------------------------------------------------------------------------
template <int BITS>
__device__ __forceinline__ void up_tile(const ChunkArgs& a, _Float16* lds, const _Float16* const* arows,
                                        const uint8_t* wq, const uint16_t* ws, int inter, int jb,
                                        _Float16* hout, const int* hrow, int cnt) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = jb * 128 + wave * 32 + (lane & 31);
  const size_t rb = (size_t)a.H * BITS / 8;
  const size_t ng = a.H / kGroup;
  const bool ok = j < inter;
  const uint8_t* brow[2] = {ok ? wq + (size_t)j * rb : nullptr, ok ? wq + (size_t)(inter + j) * rb : nullptr};
  const uint16_t* bsc[2] = {ws + (size_t)(ok ? j : 0) * ng, ws + (size_t)(ok ? inter + j : 0) * ng};
  f16v acc[2] = {};
  tile_gemm<BITS, 2>(lds, arows, a.H, brow, bsc, acc);
  if (!ok) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = acc_row(i);
    if (m < cnt) hout[(size_t)hrow[m] * inter + j] = (_Float16)(silu_f(acc[0][i]) * acc[1][i]);
  }
}

__global__ __launch_bounds__(256) void up_gemm_kernel(ChunkArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[kBM * kLdsStride];
  __shared__ const _Float16* arows[kBM];
  __shared__ int hrow[kBM];
  const int n_routed = a.route_tiles ? *a.n_tiles : 0;
  const int n_shared = a.shared_tiles;
  const int tile = blockIdx.x;
  if (tile >= n_routed + n_shared) return;
  const _Float16* xh = reinterpret_cast<const _Float16*>(a.x);
  if (tile < n_routed) {
    const int4 td = a.tiles[tile];
    const int e = td.x, r0 = td.y, cnt = td.z;
    if ((int)blockIdx.y * 128 >= a.I) return;
    if (threadIdx.x < kBM) {
      const int m = threadIdx.x;
      const int p = m < cnt ? a.sorted_pair[r0 + m] : -1;
      arows[m] = p >= 0 ? xh + (size_t)(p / a.k) * a.H : nullptr;
      hrow[m] = r0 + m;
    }
    __syncthreads();
    up_tile<4>(a, lds, arows, a.w13_q + (size_t)e * 2 * a.I * (a.H / 2), a.w13_s + (size_t)e * 2 * a.I * (a.H / kGroup),
               a.I, blockIdx.y, a.h, hrow, cnt);
  } else {
    const int t0 = (tile - n_routed) * kBM;
    const int cnt = min(kBM, a.T - t0);
    if ((int)blockIdx.y * 128 >= a.Is) return;
    if (threadIdx.x < kBM) {
      const int m = threadIdx.x;
      arows[m] = m < cnt ? xh + (size_t)(t0 + m) * a.H : nullptr;
      hrow[m] = t0 + m;
    }
    __syncthreads();
    up_tile<8>(a, lds, arows, reinterpret_cast<const uint8_t*>(a.sh13_q), a.sh13_s, a.Is, blockIdx.y, a.hs, hrow,
               cnt);
  }
}

// ---------------------------------------------------------------------------
// 5. down GEMM: y[row][n] = w_row * (h_row . W_down[n]); shared tiles write
// ys[t][n] = sigma_t * (h_s[t] . S_down[n]).  blockIdx.y: block of 256 outputs.
// ---------------------------------------------------------------------------
template <int BITS>
__device__ __forceinline__ void down_tile(const ChunkArgs& a, _Float16* lds, const _Float16* const* arows,
                                          const uint8_t* wq, const uint16_t* ws, int K, int nb, float* yout,
                                          const int* yrow, const float* yscale, int cnt) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t rb = (size_t)K * BITS / 8;
  const size_t ng = K / kGroup;
  int n[2];
  const uint8_t* brow[2];
  const uint16_t* bsc[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    n[f] = nb * 256 + wave * 64 + f * 32 + (lane & 31);
    const bool ok = n[f] < a.H;
    brow[f] = ok ? wq + (size_t)n[f] * rb : nullptr;
    bsc[f] = ws + (size_t)(ok ? n[f] : 0) * ng;
  }
  f16v acc[2] = {};
  tile_gemm<BITS, 2>(lds, arows, K, brow, bsc, acc);
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    if (n[f] >= a.H) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = acc_row(i);
      if (m < cnt) yout[(size_t)yrow[m] * a.H + n[f]] = yscale[m] * acc[f][i];
    }
  }
}

__global__ __launch_bounds__(256) void down_gemm_kernel(ChunkArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[kBM * kLdsStride];
  __shared__ const _Float16* arows[kBM];
  __shared__ int yrow[kBM];
  __shared__ float yscale[kBM];
  const int n_routed = a.route_tiles ? *a.n_tiles : 0;
  const int n_shared = a.shared_tiles;
  const int tile = blockIdx.x;
  if (tile >= n_routed + n_shared) return;
  if ((int)blockIdx.y * 256 >= a.H) return;
  if (tile < n_routed) {
    const int4 td = a.tiles[tile];
    const int e = td.x, r0 = td.y, cnt = td.z;
    if (threadIdx.x < kBM) {
      const int m = threadIdx.x;
      const int p = m < cnt ? a.sorted_pair[r0 + m] : -1;
      arows[m] = p >= 0 ? a.h + (size_t)(r0 + m) * a.I : nullptr;
      yrow[m] = r0 + m;
      yscale[m] = p >= 0 ? a.wts[p] : 0.f;
    }
    __syncthreads();
    down_tile<4>(a, lds, arows, a.w2_q + (size_t)e * a.H * (a.I / 2), a.w2_s + (size_t)e * a.H * (a.I / kGroup), a.I,
                 blockIdx.y, a.y, yrow, yscale, cnt);
  } else {
    const int t0 = (tile - n_routed) * kBM;
    const int cnt = min(kBM, a.T - t0);
    if (threadIdx.x < kBM) {
      const int m = threadIdx.x;
      arows[m] = m < cnt ? a.hs + (size_t)(t0 + m) * a.Is : nullptr;
      yrow[m] = t0 + m;
      yscale[m] = m < cnt ? a.sigma[t0 + m] : 0.f;
    }
    __syncthreads();
    down_tile<8>(a, lds, arows, reinterpret_cast<const uint8_t*>(a.sh2_q), a.sh2_s, a.Is, blockIdx.y, a.ys, yrow,
                 yscale, cnt);
  }
}

// ---------------------------------------------------------------------------
// 6. combine: out[t][n] = sum_i y[pos(t,i)][n] (+ ys[t][n]); 4 outputs/thread
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(ChunkArgs a) {
  const int t = blockIdx.y;
  const int n = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (n >= a.H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (a.ys) acc = *reinterpret_cast<const float4*>(a.ys + (size_t)t * a.H + n);
  for (int i = 0; i < a.k; ++i) {
    const int pos = a.pos_of_pair[(size_t)t * a.k + i];
    if (pos < 0) continue;
    const float4 v = *reinterpret_cast<const float4*>(a.y + (size_t)pos * a.H + n);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  const _Float16 o[4] = {(_Float16)acc.x, (_Float16)acc.y, (_Float16)acc.z, (_Float16)acc.w};
  *reinterpret_cast<uint2*>(a.out + (size_t)t * a.H + n) = *reinterpret_cast<const uint2*>(o);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int launch_route_chunk(const ChunkArgs& a, hipStream_t s) {
  dim3 g1((a.T + kBM - 1) / kBM, (a.E + 1 + 127) / 128);
  hipLaunchKernelGGL(router_gemm_kernel, g1, dim3(256), 0, s, a);
  hipLaunchKernelGGL(topk_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

int launch_experts_chunk(const ChunkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(1024), 0, s, a);
  const int max_tiles = a.max_route_tiles + a.shared_tiles;
  const int nbi = (max(a.I, a.shared_tiles ? a.Is : 0) + 127) / 128;
  hipLaunchKernelGGL(up_gemm_kernel, dim3(max_tiles, nbi), dim3(256), 0, s, a);
  hipLaunchKernelGGL(down_gemm_kernel, dim3(max_tiles, (a.H + 255) / 256), dim3(256), 0, s, a);
  hipLaunchKernelGGL(combine_kernel, dim3((a.H / 4 + 255) / 256, a.T), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace moe
