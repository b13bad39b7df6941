// Few-token path of the routed MoE block (T <= 4): one persistent launch.
//
// The block (the Chimera notebook, section 5): out = routed + sigmoid(x . W_sg)
// * shared, where the routed part is the renormalised top-k mixture of int4
// SwiGLU experts (section 5.2 ordering: softmax -> top-k -> renormalise) and
// the router rows are int8 group-64 rows stacked with the shared-gate row (the
// TensorFold PR, "Design").
//
// Work layout.  Block b belongs to group g = b % 8 (the dispatcher places it on
// XCD g) as member j = b / 8 of nj.  Group g owns the (token, slot) pairs
// p = 8q + g and slice g of the shared expert's intermediate columns, so the
// hand-off of SwiGLU activations stays among the group's members:
//   A  router rows (all groups, spread over every block) and the group's
//      shared gate/up columns       -> logits (one copy per group), shared h slice
//   R  every block ranks the logits in its group's copy (top-k, renormalised
//      weights, sigmoid gate); the ranking is deterministic, so all blocks
//      agree on the pairs without a further hand-off
//   B  the group's pairs: gate/up columns (member j: its share of the I
//      columns)                                     -> routed h
//   C  member j: output rows [j rw, (j+1) rw) of the group's partial sum
//      (its pairs' down rows and its shared slice's down rows)
//   D  the 8 partial sums of a row block are added, in group order, by member
//      j of group j % 8 and written as binary16.
//
// Hand-offs.  Values pass between blocks as 64-bit words (call tag << 32 |
// value bits) written and read with device-scope (sc1) atomic accesses; a
// reader polls the words themselves until every tag equals this call's tag,
// so no counter or flag sits between producer and consumer, and nothing has
// to be cleared after a call.  The tag is the call number: every block adds
// to its group's 64-bit call counter once, the additions of one call sum to
// kJoinQuantum, so floor(counter / kJoinQuantum) read by any block of a call
// is that call's number.  Each polled region is read by the blocks of one
// group at most: a group's copy of the logits and its activations by its nj
// members, a row block's 8 partial sums by one block.  Only a layer's output,
// with several layers per launch, is read by every block (two binary16
// outputs a word, to halve that poll).  A wave that polls waits for every
// load it has in flight (the load counter is in order), so the big weight
// loads are issued after the polls that precede them, and loads meant to stay
// in flight across a poll are held by waves that do not poll.
//
// Every wait is bounded.  A block whose wait gives up (its producers were not
// running) publishes NaN in place of the values it could not compute and
// counts itself in the workspace's give-up word, so the call's output is NaN
// rather than silently wrong, and the workspace stays consistent for the next
// call.
#include "decode.hpp"
#include "gemv.hpp"

namespace moe {

// ------------------------------------------------------------------ helpers

static constexpr uint32_t kSpinLimit = 1u << 20;  // polls before a wait gives up (about a second)

__device__ __forceinline__ void put_tagged(uint64_t* p, uint32_t tag, uint32_t bits) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_tagged_f(uint64_t* p, uint32_t tag, float v) {
  put_tagged(p, tag, __builtin_bit_cast(uint32_t, v));
}
__device__ __forceinline__ uint64_t get_tagged(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_ok(uint64_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }
__device__ __forceinline__ float word_f(uint64_t w) { return __builtin_bit_cast(float, (uint32_t)w); }

// dst[c] = sum of the 32 halves src[32 c .. 32 c + 31], c < n, in index order
__device__ __forceinline__ void chunk_sums(float* dst, const _Float16* src, int n) {
  for (int c = threadIdx.x; c < n; c += blockDim.x) {
    const h8* v = reinterpret_cast<const h8*>(src) + 4 * (size_t)c;
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const h8 w = v[q];
#pragma unroll
      for (int i = 0; i < 8; ++i) s += (float)w[i];
    }
    dst[c] = s;
  }
}

// copy n halves (n multiple of 8) global -> LDS with 16-byte accesses
__device__ __forceinline__ void copy_halves(_Float16* dst, const void* src, int n) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(dst);
  for (int i = threadIdx.x; i < n / 8; i += blockDim.x) d[i] = s[i];
}

// Wave-level poll of n tagged words w[idx(i)], i < n (word i = lane + 64 u is
// this lane's u-th): calls use(u, i, word) once every word carries the tag.
// Returns false when the wait gives up (then use() is called with NaN words).
template <int MAXW, typename Idx, typename Use>
__device__ __forceinline__ bool wave_poll(const uint64_t* w, int n, uint32_t tag, bool give_up, Idx idx, Use use) {
  const int lane = threadIdx.x & 63;
  uint64_t v[MAXW];
  bool ok = false;
  if (!give_up) {
    for (uint32_t spin = 0; spin < kSpinLimit; ++spin) {
      bool mine = true;
#pragma unroll
      for (int u = 0; u < MAXW; ++u) {
        const int i = lane + 64 * u;
        v[u] = i < n ? get_tagged(w + idx(i)) : 0;
      }
#pragma unroll
      for (int u = 0; u < MAXW; ++u)
        if (lane + 64 * u < n) mine &= tag_ok(v[u], tag);
      if (__ballot(!mine) == 0) {
        ok = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
#pragma unroll
  for (int u = 0; u < MAXW; ++u) {
    const int i = lane + 64 * u;
    if (i < n) use(u, i, ok ? v[u] : (uint64_t)0x7FC00000u);  // NaN on give-up
  }
  return ok;
}

// the arguments of layer l: every weight and gain array l strides on, the
// layer's own tagged zones
__device__ __forceinline__ DecodeArgs layer_args(const DecodeArgs& a0, int l) {
  DecodeArgs a = a0;
  if (l == 0) return a;
  const long long off = a0.lstride * l;
  auto mv = [off](auto* ptr) {
    using P = decltype(ptr);
    return ptr ? reinterpret_cast<P>(reinterpret_cast<uintptr_t>(ptr) + off) : ptr;
  };
  a.router_q = mv(a0.router_q); a.router_s = mv(a0.router_s);
  a.w13_q = mv(a0.w13_q); a.w13_s = mv(a0.w13_s);
  a.w2_q = mv(a0.w2_q); a.w2_s = mv(a0.w2_s);
  a.sh13_q = mv(a0.sh13_q); a.sh13_s = mv(a0.sh13_s);
  a.sh2_q = mv(a0.sh2_q); a.sh2_s = mv(a0.sh2_s);
  a.w13_b = mv(a0.w13_b); a.w2_b = mv(a0.w2_b);
  a.gain = mv(a0.gain);
  a.tagged = a0.tagged + (size_t)l * a0.p.z_words;
  return a;
}

// ------------------------------------------------------------------ kernel

// HC, IC, ISC: compile-time H, I, Is (0: taken from the plan); TT: most tokens
// the instance handles (1, or kDecMaxT); AFF: the routed experts are affine
// int4 (unsigned codes, w = q s + b per group of 64).  Every phase of a launch runs once, so
// code is kept short: the per-token loops are unrolled for TT tokens only, and
// the loops that cover more rows than one wave-load holds (small grids) exist
// only in the generic instances.  CB: column batches of the gate/up rows in
// flight per wave; DB: row batches of the down rows prefetched per wave.
template <int MODE, int HC, int IC, int ISC, int TT, bool AFF>
__device__ __forceinline__ void decode_layer(const DecodeArgs& a0, int l, int L) {
  extern __shared__ uint4 smem_raw[];
  constexpr int CPL8H = HC ? (HC / 1024 > 1 ? HC / 1024 : 1) : 4;  // int8 rows of H
  constexpr int CPL4H = HC ? (HC / 2048 > 1 ? HC / 2048 : 1) : 2;  // int4 rows of H
  constexpr int CPL4I = IC ? (IC / 2048 > 1 ? IC / 2048 : 1) : 2;  // int4 rows of I
  constexpr int CB = HC ? 2 : 1;
  constexpr int DB = HC ? 2 : 1;
  __shared__ int s_ids[kDecMaxT][kMaxTopK];
  __shared__ float s_w[kDecMaxT][kMaxTopK];
  __shared__ TopkScratch s_topk[kDecMaxT];
  __shared__ int s_pe[kDecMaxT];     // expert of the group's pair q (-1: none)
  __shared__ float s_pw[kDecMaxT];   // its routing weight
  __shared__ float s_sig[kDecMaxT];  // sigmoid gate of each token
  __shared__ float s_part[kDecMaxT][kMaxGroupWgs];  // this block's output rows, per token
  __shared__ uint32_t s_tag;
  __shared__ int s_bad;
  constexpr bool BLK = MODE == DEC_BLOCK || MODE == DEC_LAYERS;  // RMSNorm in front, residual after
  __shared__ __attribute__((aligned(16))) _Float16 s_gain[BLK ? kMaxHidden : 8];
  __shared__ float s_rn[kDecMaxT];
  // With several layers, the indices are taken anew in every layer through
  // empty asm statements: otherwise the compiler hoists the body's index and
  // address arithmetic out of the loop and keeps it in registers across the
  // whole body.
  int tid_ = threadIdx.x, b_ = blockIdx.x;
  if (MODE == DEC_LAYERS) {
    asm volatile("" : "+v"(tid_));
    asm volatile("" : "+s"(b_));
  }
  const DecodeArgs al = MODE == DEC_LAYERS ? layer_args(a0, l) : DecodeArgs{};
  const DecodeArgs& a = MODE == DEC_LAYERS ? al : a0;
  const DecodePlan& p = a.p;
  const int H = HC ? HC : p.H;
  const int I = IC ? IC : p.I;
  const int Is = ISC ? ISC : p.Is;
  const int T = p.T, E = p.E, k = p.k, nb = p.nb, nj = p.nj;
  const int S = p.S, sw = p.sw;
  const int tid = tid_, wave = tid >> 6, lane = tid & 63;
  const int b = b_, g = b % kGroups, j = b / kGroups;
  _Float16* act = reinterpret_cast<_Float16*>(smem_raw);  // [T][H]
  _Float16* hq = act + (size_t)T * H;                     // [npg][I] the group's routed h
  _Float16* hs = hq + (size_t)p.npg * I;                  // [T][sw] the group's shared slice
  float* xsum = reinterpret_cast<float*>(hs + (size_t)T * sw);  // AFF: [T][H/32] chunk sums of act
  float* hsum = xsum + (size_t)T * (H / 32);                    // AFF: [npg][I/32] chunk sums of hq
  uint64_t* const zx_prev = l > 0 ? a.tagged - p.z_words + p.z_x : nullptr;  // the previous layer's output
  uint64_t* const zl = a.tagged + p.z_logits;
  uint64_t* const zs = a.tagged + p.z_hs;
  uint64_t* const zh = a.tagged + p.z_h;
  const bool give_up = a.give_up != 0;

  // ---------------- stage A loads: router rows (wave 0), shared gate/up columns (wave 1)
  const RowGeom g8h = row_geom(H, 8);
  const int r_first = b;  // router rows b, b + nb, ...
  Frag<8, 1, CPL8H> fr;
  Frag<8, 2, CPL8H> fs;
  int r_row = -1, s_col = -1;
  if (MODE != DEC_EXPERTS) {
    if (wave == 0) {
      const int r = r_first + nb * (lane / g8h.lpr);
      r_row = r <= E ? r : -1;
      const uint8_t* rows[1] = {r_row >= 0 ? reinterpret_cast<const uint8_t*>(a.router_q) + (size_t)r * H : nullptr};
      const uint16_t* srow[1] = {a.router_s + (size_t)(r_row >= 0 ? r : 0) * (H / kGroup)};
      fr.load(rows, srow, g8h, reinterpret_cast<const uint8_t*>(a.router_q));
    } else if (wave == 1 && g < S) {
      const int c = j + nj * (lane / g8h.lpr);  // column of the slice
      s_col = c < sw ? c : -1;
      const int cg = g * sw + (s_col >= 0 ? c : 0);
      const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sh13_q);
      const uint8_t* rows[2] = {s_col >= 0 ? base + (size_t)cg * H : nullptr,
                                s_col >= 0 ? base + (size_t)(Is + cg) * H : nullptr};
      const uint16_t* srow[2] = {a.sh13_s + (size_t)cg * (H / kGroup), a.sh13_s + (size_t)(Is + cg) * (H / kGroup)};
      fs.load(rows, srow, g8h, base);
    }
  }
  if (tid == 0 && l == 0) {
    // join this call: the additions of one call to each group counter sum to kJoinQuantum
    const uint64_t add = j == 0 ? kJoinQuantum - (uint64_t)(nj - 1) : 1u;
    const uint64_t before = __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(a.sync + kJoinWord + kSyncStride * g),
                                                   add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_tag = (uint32_t)(before / kJoinQuantum) + 1u;
    s_bad = 0;
  }
  if (l == 0) {
    copy_halves(act, a.x, T * H);
  } else {
    // the previous layer's output, once its reducers have published all of it
    // (the tag is read in a barrier-ordered copy: s_tag was set before layer 0's
    // barrier); word i carries outputs 2i (low half) and 2i + 1
    const uint32_t tg = s_tag;
    const int nw = T * H / 2;
    uint32_t* act2 = reinterpret_cast<uint32_t*>(act);
    for (int base = wave * 64 * 4; base < nw; base += 256 * 4) {
      const bool ok = wave_poll<4>(zx_prev + base, min(256, nw - base), tg, give_up, [](int i) { return i; },
                                   [&](int, int i, uint64_t w) { act2[base + i] = (uint32_t)w; });
      if (!ok && lane == 0) s_bad = 1;
    }
  }
  if (BLK) copy_halves(s_gain, a.gain, H);
  __syncthreads();
  const uint32_t tag = s_tag;
  // DEC_BLOCK, DEC_LAYERS (the Chimera notebook, sections 7 and 10: post-attention RMSNorm
  // in front of the block, residual after it): wave t sums token t's squares
  // in a fixed order, so every block derives the same binary16 activations.
  if (BLK) {
    if (wave < T) {
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
      h8* pp = reinterpret_cast<h8*>(act + (size_t)t * H) + c;
      const h8 gv = reinterpret_cast<const h8*>(s_gain)[c];
      h8 v = *pp;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (_Float16)((float)v[i] * s_rn[t] * ((float)gv[i] + a.gain_add));
      *pp = v;
    }
    __syncthreads();
  }

  // ---------------- stage A: publish logits and the shared slice's activations
  if (MODE != DEC_EXPERTS) {
    if (wave == 0 && r_first <= E) {
      float acc[1][TT];
      fr.template dot_shared<TT>(g8h, act, H, T, acc);
#pragma unroll
      for (int t = 0; t < TT; ++t)
        if (t < T) {
          const float v = lane_group_sum(acc[0][t], g8h.lpr);  // in every lane of the row's lanes
          if (r_row >= 0)
            for (int c = lane % g8h.lpr; c < kGroups; c += g8h.lpr)
              put_tagged_f(zl + c * p.zl_copy + (size_t)t * (E + 1) + r_row, tag, v);
        }
    }
    if (wave == 1 && g < S && j < sw) {
      float acc[2][TT];
      fs.template dot_shared<TT>(g8h, act, H, T, acc);
#pragma unroll
      for (int t = 0; t < TT; ++t)
        if (t < T) {
          const float gt = lane_group_sum(acc[0][t], g8h.lpr);
          const float up = lane_group_sum(acc[1][t], g8h.lpr);
          if (s_col >= 0 && (lane % g8h.lpr) == 0)
            put_tagged_f(zs + ((size_t)g * T + t) * sw + s_col, tag, silu_f(gt) * up);
        }
    }
    // more router rows or shared columns than one wave-load holds (small grids)
    for (int r0 = r_first + nb * g8h.rpb; HC == 0 && r0 <= E; r0 += nb * g8h.rpb) {
      if (wave != 0) break;
      const int r = r0 + nb * (lane / g8h.lpr);
      const uint8_t* rows[1] = {r <= E ? reinterpret_cast<const uint8_t*>(a.router_q) + (size_t)r * H : nullptr};
      const uint16_t* srow[1] = {a.router_s + (size_t)(r <= E ? r : 0) * (H / kGroup)};
      Frag<8, 1, CPL8H> f;
      f.load(rows, srow, g8h, reinterpret_cast<const uint8_t*>(a.router_q));
      float acc[1][TT];
      f.template dot_shared<TT>(g8h, act, H, T, acc);
#pragma unroll
      for (int t = 0; t < TT; ++t)
        if (t < T) {
          const float v = lane_group_sum(acc[0][t], g8h.lpr);
          if (r <= E)
            for (int c = lane % g8h.lpr; c < kGroups; c += g8h.lpr)
              put_tagged_f(zl + c * p.zl_copy + (size_t)t * (E + 1) + r, tag, v);
        }
    }
    for (int c0 = j + nj * g8h.rpb; HC == 0 && g < S && c0 < sw; c0 += nj * g8h.rpb) {
      if (wave != 1) break;
      const int c = c0 + nj * (lane / g8h.lpr);
      const int cg = g * sw + (c < sw ? c : 0);
      const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sh13_q);
      const uint8_t* rows[2] = {c < sw ? base + (size_t)cg * H : nullptr, c < sw ? base + (size_t)(Is + cg) * H : nullptr};
      const uint16_t* srow[2] = {a.sh13_s + (size_t)cg * (H / kGroup), a.sh13_s + (size_t)(Is + cg) * (H / kGroup)};
      Frag<8, 2, CPL8H> f;
      f.load(rows, srow, g8h, base);
      float acc[2][TT];
      f.template dot_shared<TT>(g8h, act, H, T, acc);
#pragma unroll
      for (int t = 0; t < TT; ++t)
        if (t < T) {
          const float gt = lane_group_sum(acc[0][t], g8h.lpr);
          const float up = lane_group_sum(acc[1][t], g8h.lpr);
          if (c < sw && (lane % g8h.lpr) == 0) put_tagged_f(zs + ((size_t)g * T + t) * sw + c, tag, silu_f(gt) * up);
        }
    }
  }

  // ---------------- shared down rows of this block (routing-independent), issued
  // now by waves 2 and 3, which do not poll for the routing: a wave that polls
  // waits for every load it has in flight
  // rows n in [j rw, (j+1) rw), K slice [g sw, (g+1) sw), one row batch per wave
  const RowGeom g8s = row_geom(sw, 8);
  const int n0 = j * p.rw;
  const int nsb = (p.rw + g8s.rpb - 1) / g8s.rpb;  // row batches of the shared down rows
  const bool shared_down = MODE != DEC_EXPERTS && g < S;
  Frag<8, 1, 1> fd_s;
  {
    const int rbi = wave - 2;
    const int r = rbi * g8s.rpb + lane / g8s.lpr;
    const int n = n0 + r;
    const bool ok = shared_down && rbi >= 0 && rbi < nsb && r < p.rw && n < H;
    const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sh2_q);
    const uint8_t* rows[1] = {ok ? base + (size_t)n * Is + (size_t)g * sw : nullptr};
    const uint16_t* srow[1] = {a.sh2_s + (size_t)(ok ? n : 0) * (Is / kGroup) + (size_t)g * sw / kGroup};
    if (wave >= 2) fd_s.load(rows, srow, g8s, base);
  }
  for (int t = tid; t < kDecMaxT * kMaxGroupWgs; t += blockDim.x) (&s_part[0][0])[t] = 0.f;
  // AFF: the offsets multiply the sum of each 32-activation chunk
  if (AFF) chunk_sums(xsum, act, T * (H / 32));

  // ---------------- routing: every block ranks its tokens (wave t: token t, lane
  // l: experts 4l..4l+3) from its group's copy of the logits
  if (MODE != DEC_EXPERTS) {
    if (wave < T) {
      const int t = wave;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      float gate = 0.f;
      const uint64_t* lw = zl + g * p.zl_copy + (size_t)t * (E + 1);
      // word 4 of every lane is the gate logit E; experts at or past E are ignored by the ranking
      const bool ok = wave_poll<5>(lw, 5 * 64, tag, give_up,
                                   [&](int i) { return i < 256 ? min(4 * (i % 64) + i / 64, E) : E; },
                                   [&](int u, int, uint64_t w) {
                                     if (u < 4) v[u] = word_f(w);
                                     else gate = word_f(w);
                                   });
      if (ok) {
        wave_topk(v, E, k, s_ids[t], s_w[t], s_topk[t]);
        if (lane == 0) s_sig[t] = sigmoid_f(gate);
      } else {
        if (lane < k) { s_ids[t][lane] = 0; s_w[t][lane] = __builtin_nanf(""); }
        if (lane == 0) { s_sig[t] = __builtin_nanf(""); s_bad = 1; }
      }
    }
    __syncthreads();
    for (int q = tid; q < kDecMaxT; q += blockDim.x) {
      const int pp = kGroups * q + g;
      s_pe[q] = pp < T * k ? s_ids[pp / k][pp % k] : -1;
      s_pw[q] = pp < T * k ? s_w[pp / k][pp % k] : 0.f;
    }
    if (b == nb - 1) {
      for (int q = tid; q < T * k; q += blockDim.x) {
        if (a.ids_out) a.ids_out[q] = s_ids[q / k][q % k];
        if (a.w_out) a.w_out[q] = s_w[q / k][q % k];
      }
      for (int t = tid; t < T; t += blockDim.x)
        if (a.sigma_out) a.sigma_out[t] = s_sig[t];
    }
  } else if (tid < kDecMaxT) {
    const int pp = kGroups * tid + g;
    int e = pp < T * k ? a.ids_in[pp] : -1;
    s_pe[tid] = (e >= 0 && e < E) ? e : -1;  // ids outside [0, E) contribute nothing
    s_pw[tid] = pp < T * k ? a.w_in[pp] : 0.f;
  }
  __syncthreads();
  const int np = min(p.npg, (T * k - g + kGroups - 1) / kGroups);  // pairs of this group

  // ---------------- stage B: gate/up columns of the group's pairs
  // member j: columns [j cw, (j+1) cw) of each pair, in batches of rpb columns;
  // the down rows of pair 0 are loaded with pair 0's gate/up rows
  const RowGeom g4h = row_geom(H, 4);
  const RowGeom g4i = row_geom(I, 4);
  const int c_lo = j * p.cw, c_hi = min(I, c_lo + p.cw);
  const int ncb = (c_hi - c_lo + g4h.rpb - 1) / g4h.rpb;  // column batches
  const size_t rb13 = (size_t)H / 2, ng13 = H / kGroup;
  const size_t rb2 = (size_t)I / 2, ng2 = I / kGroup;
  const int nrb = (p.rw + g4i.rpb - 1) / g4i.rpb;  // row batches of the down rows
  Frag<4, DB, CPL4I, AFF> fd0;
  {  // (no branch: a branch here would make the compiler wait for these loads inside it)
    const int e = np > 0 && s_pe[0] >= 0 ? s_pe[0] : 0;
    const uint8_t* rows[DB];
    const uint16_t* srow[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      const int rbi = wave + 4 * d;
      const int r = rbi * g4i.rpb + lane / g4i.lpr;
      const int n = n0 + r;
      const bool ok = np > 0 && rbi < nrb && r < p.rw && n < H;
      rows[d] = ok ? a.w2_q + ((size_t)e * H + n) * rb2 : nullptr;
      srow[d] = a.w2_s + ((size_t)e * H + (ok ? n : 0)) * ng2;
    }
    fd0.load(rows, srow, g4i, a.w2_q);
    if (AFF) {
      const uint16_t* orow[DB];
#pragma unroll
      for (int d = 0; d < DB; ++d) orow[d] = a.w2_b + (srow[d] - a.w2_s);
      fd0.load_offsets(orow, g4i);
    }
  }
  for (int q = 0; q < np; ++q) {
    const int e = s_pe[q];
    if (e < 0) continue;  // uniform
    const int t = (kGroups * q + g) / k;
    for (int cb0 = wave; cb0 < ncb; cb0 += 4 * CB) {
      const uint8_t* rows[2 * CB];
      const uint16_t* srow[2 * CB];
      int col[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const int cb = cb0 + 4 * u;
        const int c = c_lo + cb * g4h.rpb + lane / g4h.lpr;
        const bool ok = cb < ncb && c < c_hi;
        col[u] = ok ? c : -1;
        const size_t rg = (size_t)e * 2 * I + (ok ? c : 0), ru = rg + I;
        rows[u] = ok ? a.w13_q + rg * rb13 : nullptr;
        rows[CB + u] = ok ? a.w13_q + ru * rb13 : nullptr;
        srow[u] = a.w13_s + rg * ng13;
        srow[CB + u] = a.w13_s + ru * ng13;
      }
      Frag<4, 2 * CB, CPL4H, AFF> f;
      f.load(rows, srow, g4h, a.w13_q);
      if (AFF) {
        const uint16_t* orow[2 * CB];
#pragma unroll
        for (int u = 0; u < 2 * CB; ++u) orow[u] = a.w13_b + (srow[u] - a.w13_s);
        f.load_offsets(orow, g4h);
      }
      float acc[2 * CB][1];
      f.template dot_shared<1>(g4h, act + (size_t)t * H, H, 1, acc, xsum + (size_t)t * (H / 32), 0);
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const float gt = lane_group_sum(acc[u][0], g4h.lpr);
        const float up = lane_group_sum(acc[CB + u][0], g4h.lpr);
        // staged in the LDS rows the gather below fills (with the same binary16 value)
        if (col[u] >= 0 && (lane % g4h.lpr) == 0) hq[(size_t)q * I + col[u]] = (_Float16)(silu_f(gt) * up);
      }
    }
  }
  // Publish this member's columns: consecutive lanes write consecutive words,
  // so each member's run leaves as whole pieces of lines rather than one
  // 8-byte store per column (single-word stores from several waves took
  // microseconds longer to become visible).  Then wait for the acknowledgement
  // of this block's own stores before polling the other members' words.
  __syncthreads();
  for (int q = 0; q < np; ++q) {
    if (s_pe[q] < 0) continue;  // uniform
    for (int c = c_lo + tid; c < c_hi; c += blockDim.x)
      put_tagged_f(zh + ((size_t)g * p.npg + q) * I + c, tag,
                   s_bad ? __builtin_nanf("") : (float)hq[(size_t)q * I + c]);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---------------- the group's routed activations (pairs with an expert only:
  // nothing is written for a dropped pair) and its shared slice -> LDS
  for (int q = 0; q < np; ++q) {
    if (s_pe[q] < 0) continue;
    for (int base = wave * 64 * 4; base < I; base += 256 * 4) {
      const bool ok = wave_poll<4>(zh + ((size_t)g * p.npg + q) * I + base, min(256, I - base), tag, give_up,
                                   [](int i) { return i; },
                                   [&](int, int i, uint64_t w) { hq[(size_t)q * I + base + i] = (_Float16)word_f(w); });
      if (!ok && lane == 0) s_bad = 1;
    }
  }
  if (shared_down) {
    const int n = T * sw;
    for (int base = wave * 64 * 4; base < n; base += 256 * 4) {
      const bool ok = wave_poll<4>(zs + (size_t)g * T * sw + base, min(256, n - base), tag, give_up,
                                   [](int i) { return i; },
                                   [&](int, int i, uint64_t w) { hs[base + i] = (_Float16)word_f(w); });
      if (!ok && lane == 0) s_bad = 1;
    }
  }
  __syncthreads();
  if (AFF) {
    chunk_sums(hsum, hq, np * (I / 32));
    if (!shared_down) __syncthreads();  // otherwise the shared down's barrier orders it
  }

  // ---------------- shared down: sigma * (this block's rows over the group's slice)
  if (shared_down) {
    for (int rbi = wave - 2, m = 0; wave >= 2 && rbi < nsb; rbi += 2, ++m) {
      const int r = rbi * g8s.rpb + lane / g8s.lpr;
      const int n = n0 + r;
      const bool ok = r < p.rw && n < H;
      Frag<8, 1, 1> f;
      if (m == 0) {
        f = fd_s;
      } else {
        const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sh2_q);
        const uint8_t* rows[1] = {ok ? base + (size_t)n * Is + (size_t)g * sw : nullptr};
        const uint16_t* srow[1] = {a.sh2_s + (size_t)(ok ? n : 0) * (Is / kGroup) + (size_t)g * sw / kGroup};
        f.load(rows, srow, g8s, base);
      }
      float acc[1][TT];
      f.template dot_shared<TT>(g8s, hs, sw, T, acc);
#pragma unroll
      for (int t = 0; t < TT; ++t)
        if (t < T) {
          const float v = lane_group_sum(acc[0][t], g8s.lpr);
          if (ok && (lane % g8s.lpr) == 0) s_part[t][r] = s_sig[t] * v;
        }
    }
    __syncthreads();
  }

  // ---------------- down rows of the group's pairs, weighted, into this block's rows
  for (int q = 0; q < np; ++q) {
    const int e = s_pe[q];
    if (e < 0) continue;
    const int t = (kGroups * q + g) / k;
    const float wq = s_pw[q];
    for (int rb0 = wave; rb0 < nrb; rb0 += 4 * DB) {
      Frag<4, DB, CPL4I, AFF> f;
      if (q == 0 && rb0 == wave) {
        f = fd0;
      } else {
        const uint8_t* rows[DB];
        const uint16_t* srow[DB];
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          const int rbi = rb0 + 4 * d;
          const int r = rbi * g4i.rpb + lane / g4i.lpr;
          const int n = n0 + r;
          const bool ok = rbi < nrb && r < p.rw && n < H;
          rows[d] = ok ? a.w2_q + ((size_t)e * H + n) * rb2 : nullptr;
          srow[d] = a.w2_s + ((size_t)e * H + (ok ? n : 0)) * ng2;
        }
        f.load(rows, srow, g4i, a.w2_q);
        if (AFF) {
          const uint16_t* orow[DB];
#pragma unroll
          for (int d = 0; d < DB; ++d) orow[d] = a.w2_b + (srow[d] - a.w2_s);
          f.load_offsets(orow, g4i);
        }
      }
      const _Float16* hv[DB];
      const float* hx[DB];
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        hv[d] = hq + (size_t)q * I;
        hx[d] = hsum + (size_t)q * (I / 32);
      }
      float acc[DB];
      f.dot_per_batch(g4i, hv, acc, hx);
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const float y = lane_group_sum(acc[d], g4i.lpr);
        const int r = (rb0 + 4 * d) * g4i.rpb + lane / g4i.lpr;
        if (rb0 + 4 * d < nrb && r < p.rw && (lane % g4i.lpr) == 0) s_part[t][r] += wq * y;
      }
    }
    __syncthreads();  // pairs of one token add into the same rows
  }

  // ---------------- the row block's sum over the 8 groups
  // Every member publishes its rows of the group's partial sum; the member j of
  // group j % 8 waits for the 8 partial sums of its rows, adds them in group
  // order and writes the output.
  __syncthreads();
  uint64_t* const zp = a.tagged + p.z_part;
  for (int q = tid; q < T * p.rw; q += blockDim.x) {
    const int t = q / p.rw, r = q - t * p.rw;
    if (n0 + r < H)
      put_tagged_f(zp + ((size_t)g * T + t) * H + n0 + r, tag, s_bad ? __builtin_nanf("") : s_part[t][r]);
  }
  if (g == j % kGroups) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this block's own partial sums acknowledged first
    const int t = tid / p.rw, r = tid - t * p.rw, n = n0 + r;
    const bool mine = tid < T * p.rw && n < H;  // T * rw <= 256: one output per thread
    uint64_t v[kGroups];
    bool ok = false;
    if (!give_up) {
      for (uint32_t spin = 0; spin < kSpinLimit; ++spin) {
        bool got = true;
#pragma unroll
        for (int gg = 0; gg < kGroups; ++gg) v[gg] = mine ? get_tagged(zp + ((size_t)gg * T + t) * H + n) : 0;
#pragma unroll
        for (int gg = 0; gg < kGroups; ++gg) got &= !mine || tag_ok(v[gg], tag);
        if (__ballot(!got) == 0) {
          ok = true;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    uint32_t o = 0;
    if (mine) {
      // DEC_BLOCK, DEC_LAYERS: the residual stream (layer l >= 1: the previous layer's
      // output, whose words this block has already seen complete)
      float sum = 0.f;
      if (BLK) {
        uint16_t rb = 0;
        if (l == 0) {
          rb = a.x[(size_t)t * H + n];
        } else {
          const uint32_t w = (uint32_t)get_tagged(zx_prev + ((size_t)t * H + n) / 2);
          rb = (uint16_t)(n & 1 ? w >> 16 : w);
        }
        sum = half_bits_to_float(rb);
      }
#pragma unroll
      for (int gg = 0; gg < kGroups; ++gg) sum += word_f(v[gg]);
      o = __builtin_bit_cast(uint16_t, (_Float16)(ok ? sum : __builtin_nanf("")));
      if (l == L - 1) a.out[(size_t)t * H + n] = (uint16_t)o;
    }
    if (l < L - 1) {
      // outputs n (even) and n + 1 share one word: rw is even, so they are
      // this thread's and the next one's
      const uint32_t o_next = (uint32_t)__shfl_xor((int)o, 1, 64);
      if (mine && (n & 1) == 0) put_tagged(a.tagged + p.z_x + ((size_t)t * H + n) / 2, tag, o | (o_next << 16));
    }
    if (!ok && lane == 0) s_bad = 1;
  }
  __syncthreads();
  if (l == L - 1 && threadIdx.x == 0 && s_bad)
    __hip_atomic_fetch_add(a0.sync + kGiveUpWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MODE, int HC, int IC, int ISC, int TT, bool AFF>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a0) {
  // DEC_LAYERS applies L sub-blocks in turn (the Chimera notebook, "Pipeline":
  // every layer's weights at one fixed offset from the previous layer's); a
  // layer's output reaches every block of the next one through the tagged
  // words of its x zone.  The other modes run one layer.
  if (MODE == DEC_LAYERS) {
    for (int l = 0; l < a0.L; ++l) decode_layer<MODE, HC, IC, ISC, TT, AFF>(a0, l, a0.L);
  } else {
    decode_layer<MODE, HC, IC, ISC, TT, AFF>(a0, 0, 1);
  }
}

// ------------------------------------------------------------------ host side

bool decode_real_widths(int H, int I, int Is) { return H == 2048 && I == 512 && Is == 512; }

// the kernel instance of a mode and widths for a variant (decode_variant)
template <int MODE, int HC, int IC, int ISC>
static const void* kernel_of(int variant) {
  switch (variant) {
    case 0: return reinterpret_cast<const void*>(&decode_kernel<MODE, HC, IC, ISC, 1, false>);
    case 1: return reinterpret_cast<const void*>(&decode_kernel<MODE, HC, IC, ISC, kDecMaxT, false>);
    case 2: return reinterpret_cast<const void*>(&decode_kernel<MODE, HC, IC, ISC, 1, true>);
    default: return reinterpret_cast<const void*>(&decode_kernel<MODE, HC, IC, ISC, kDecMaxT, true>);
  }
}

template <int MODE>
static const void* kernel_of(bool real, int variant) {
  return real ? kernel_of<MODE, 2048, 512, 512>(variant) : kernel_of<MODE, 0, 0, 0>(variant);
}

static const void* kernel_of(int mode, bool real, int variant) {
  if (mode == DEC_BLOCK) return kernel_of<DEC_BLOCK>(real, variant);
  if (mode == DEC_LAYERS) return kernel_of<DEC_LAYERS>(real, variant);
  return mode == DEC_FORWARD ? kernel_of<DEC_FORWARD>(real, variant) : kernel_of<DEC_EXPERTS>(real, variant);
}

int decode_blocks_per_cu(int mode, bool real, int variant, size_t lds_bytes) {
  int n = 0;
  const hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel_of(mode, real, variant), 256, lds_bytes);
  return err == hipSuccess ? n : 0;
}

int launch_decode(const DecodeArgs& a, int mode, bool real, size_t lds_bytes, hipStream_t s) {
  if (real && (!decode_real_widths(a.p.H, a.p.I, a.p.Is) || a.p.nj != kMaxGroupWgs)) return MOE_ERR_LAUNCH;
  const void* k = kernel_of(mode, real, decode_variant(a.p.T, a.affine != 0));
  void* args[] = {const_cast<DecodeArgs*>(&a)};
  return hipLaunchKernel(k, dim3(a.p.nb), dim3(256), args, lds_bytes, s) == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace moe
