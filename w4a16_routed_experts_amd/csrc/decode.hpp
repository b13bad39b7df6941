// Arguments and launcher of the few-token path (T <= 4): one persistent launch.
#pragma once
#include "common.hpp"

namespace moe {

static constexpr int kDecMaxT = 4;        // tokens per call on this path
static constexpr int kGroups = 8;         // workgroup groups (block b is in group b % 8, one per XCD)
static constexpr int kMaxGroupWgs = 64;   // workgroups per group at most (grid <= 512)
static constexpr int kSyncStride = 32;    // counters 128 bytes apart (in 32-bit words)
static constexpr int kCounterPages = 2;   // words [0, 2048) of the sync area: path counters
static constexpr int kFlagPage = 1024;    // words per page
static constexpr int kSyncBytes = (kCounterPages + 8) * kFlagPage * 4;  // 40 KiB, zero between calls
static constexpr int kMaxHidden = 4096;   // widest admitted hidden size
static constexpr int kMaxLayers = 256;    // sub-blocks per call at most (moe_layers_forward)
// DEC_BLOCK: the forward with RMSNorm in front and the residual after;
// DEC_LAYERS: DEC_BLOCK applied to L layers in turn
enum { DEC_FORWARD = 0, DEC_EXPERTS = 1, DEC_BLOCK = 2, DEC_LAYERS = 3 };
static constexpr int kDecModes = 4;

// Sync-area words used by the few-token path (the grouped-GEMM path uses the
// word at kCounterPages * kFlagPage - kSyncStride).
static constexpr int kJoinWord = 0;                       // 8 call counters (64-bit), one line each
static constexpr int kGiveUpWord = 8 * kSyncStride;       // count of workgroups whose bounded wait gave up
static constexpr uint64_t kJoinQuantum = 1u << 16;        // each call adds exactly this to every call counter

// Work decomposition; the host and the kernel both use these numbers.
struct DecodePlan {
  int T, H, E, k, I, Is;
  int nb, nj;     // grid, workgroups per group (nb / 8)
  int S;          // shared-expert slices: 8 (one per group) or 1 (group 0 takes it all)
  int sw;         // shared intermediate columns per slice (Is / S)
  int npg;        // routed (token, slot) pairs per group at most: ceil(T k / 8)
  int cw;         // routed intermediate columns per workgroup and pair: ceil(I / nj)
  int rw;         // output rows per workgroup: ceil(H / nj), rounded up to even
  int scw;        // shared columns per workgroup: ceil(sw / nj)
  // tagged zones (64-bit words: call tag << 32 | value bits)
  size_t z_logits;  // [8][T][E + 1]: one copy of the logits per group, zl_copy words apart
  size_t zl_copy;
  size_t z_hs;      // [8][T][sw] shared SwiGLU activations of each slice
  size_t z_h;       // [8][npg][I] routed SwiGLU activations of each group's pairs
  size_t z_part;    // [8][T][H] each group's partial output rows
  size_t z_x;       // [T][H/2] the layer's output (two binary16 values a word), read by every block of the next layer
  size_t z_words;   // tagged words of one layer (each layer of a call has its own zones)
};

__host__ __device__ inline DecodePlan decode_plan(int H, int E, int k, int I, int Is, int T, int nb) {
  DecodePlan p;
  p.T = T; p.H = H; p.E = E; p.k = k; p.I = I; p.Is = Is;
  p.nb = nb;
  p.nj = nb / kGroups;
  p.S = (Is / kGroups) % 16 == 0 ? kGroups : 1;
  p.sw = Is / p.S;
  p.npg = (T * k + kGroups - 1) / kGroups;
  p.cw = (I + p.nj - 1) / p.nj;
  p.rw = ((H + p.nj - 1) / p.nj + 1) & ~1;  // even: a layer's output words carry two outputs
  p.scw = (p.sw + p.nj - 1) / p.nj;
  size_t o = 0;
  p.zl_copy = ((size_t)T * (E + 1) + 15) / 16 * 16;
  p.z_logits = o; o += kGroups * p.zl_copy;
  p.z_hs = o; o += (size_t)kGroups * T * p.sw;
  o = (o + 15) / 16 * 16;
  p.z_h = o; o += (size_t)kGroups * p.npg * I;
  o = (o + 15) / 16 * 16;
  p.z_part = o; o += (size_t)kGroups * T * H;
  o = (o + 15) / 16 * 16;
  p.z_x = o; o += (size_t)T * H / 2;
  p.z_words = (o + 15) / 16 * 16;
  return p;
}

// dynamic LDS of one workgroup: activations [T][H], the group's routed h
// [npg][I] and its shared slice [T][sw], all binary16, then (affine experts)
// float sums of every 32 consecutive activations of each: [T][H/32], [npg][I/32]
__host__ __device__ inline size_t decode_lds_bytes(const DecodePlan& p) {
  return ((size_t)p.T * p.H + (size_t)p.npg * p.I + (size_t)p.T * p.sw) * 2 +
         ((size_t)p.T * (p.H / 32) + (size_t)p.npg * (p.I / 32)) * 4;
}

struct DecodeArgs {
  const int8_t* router_q; const uint16_t* router_s;
  const uint8_t* w13_q; const uint16_t* w13_s;
  const uint8_t* w2_q; const uint16_t* w2_s;
  const int8_t* sh13_q; const uint16_t* sh13_s;
  const int8_t* sh2_q; const uint16_t* sh2_s;
  const uint16_t* x;
  uint16_t* out;
  const uint16_t* gain;  // DEC_BLOCK, DEC_LAYERS: RMSNorm gain [H] (x is the residual stream)
  float eps;             // DEC_BLOCK, DEC_LAYERS: RMSNorm epsilon
  float gain_add;        // added to every gain element in fp32 (1: the gain holds w of 1 + w)
  int32_t* ids_out; float* w_out; float* sigma_out;  // nullable
  const int32_t* ids_in; const float* w_in;          // routing given by the caller
  uint32_t* sync;        // the workspace's sync area (kSyncBytes)
  uint64_t* tagged;      // tagged zones (L x plan.z_words words)
  int give_up;           // nonzero: every bounded wait gives up at once (exercises the failure path)
  int affine;            // routed experts are affine int4 (unsigned codes, w = q s + b)
  const uint16_t* w13_b; const uint16_t* w2_b;  // affine: per-group binary16 offsets
  int L;                 // DEC_LAYERS: sub-blocks applied in turn (1 otherwise)
  long long lstride;     // bytes from one layer's weight (and gain) arrays to the next layer's
  DecodePlan p;
};


// kernel instances: by token count (1, or up to kDecMaxT) and weight format
static constexpr int kDecVariants = 4;
__host__ __device__ inline int decode_variant(int T, bool affine) { return (T == 1 ? 0 : 1) + (affine ? 2 : 0); }
int decode_blocks_per_cu(int mode, bool real_widths, int variant, size_t lds_bytes);
// real: the instance built for H = 2048, I = Is = 512, which needs
// p.nj == kMaxGroupWgs (it has no loop for a second router row or shared
// column per member)
int launch_decode(const DecodeArgs& a, int mode, bool real, size_t lds_bytes, hipStream_t s);
bool decode_real_widths(int H, int I, int Is);

}  // namespace moe
