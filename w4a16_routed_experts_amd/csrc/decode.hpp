// Arguments and launcher of the few-token (persistent GEMV) path.
#pragma once
#include "common.hpp"

namespace moe {

static constexpr int kDecMaxT = 4;        // tokens per call on this path
static constexpr int kSyncStride = 32;    // counters 128 bytes apart (in 32-bit words)
static constexpr int kXcds = 8;           // XCDs of an MI355X
static constexpr int kFlagPage = 1024;    // per-XCD flag pages 4 KiB apart (in words)
static constexpr int kCounterPages = 2;   // 64 counter slots
static constexpr int kSubCounters = 8;    // items of a stage count on 8 sub-counters, then one top counter
static constexpr int kSyncBytes = (kCounterPages + kXcds) * kFlagPage * 4;  // counters, then one flag page per XCD
enum { SYNC_ROUTER = 0, SYNC_SHUP = 1, SYNC_UP = 2, SYNC_SD = 3, SYNC_EXIT = 4, SYNC_ERR = 5, SYNC_COUNT = 6 };
enum { DEC_FORWARD = 0, DEC_EXPERTS = 1, DEC_BLOCK = 2 };  // DEC_BLOCK: the forward with RMSNorm and residual
static constexpr int kDecModes = 3;
static constexpr int kMaxHidden = 4096;  // widest admitted hidden size

__host__ __device__ constexpr int round32(int x) { return (x + 31) / 32 * 32; }

// rows of a K-wide row that one 64-lane load covers (16-byte chunks per lane)
__host__ __device__ constexpr int rows_per_load(int K, int bits) {
  return 64 / ((K * bits / 128) < 64 ? (K * bits / 128) : 64);
}

// Work decomposition of the few-token path; the host and the kernel both use
// these numbers.  Every item writes its results to its own 128-byte-aligned
// region of the workspace (floats), so no cache line is shared by producers.
struct DecodePlan {
  int n_router, n_shup, n_up, n_sd, n_down;
  int up_jblocks;           // j-blocks per (token, slot)
  int lg_rows, lg_stride;   // router rows per item; floats per (item, token)
  int hs_cols, hs_stride;   // shared gate/up columns per item; floats per (item, token)
  int he_cols, he_stride;   // expert gate/up columns per item; floats (4-byte units) per item
  int ss_rows, ss_stride;   // shared down rows per item; floats per (item, token)
  int down_rows;            // output rows per down item
};

__host__ __device__ inline DecodePlan decode_plan(int H, int E, int k, int I, int Is, int T, bool routed_only) {
  DecodePlan p;
  const int r8h = rows_per_load(H, 8), r4h = rows_per_load(H, 4), r8s = rows_per_load(Is, 8);
  p.lg_rows = 4 * r8h;
  p.hs_cols = 8 * r8h;
  p.he_cols = 16 * r4h;
  p.ss_rows = 16 * r8s;
  p.lg_stride = round32(p.lg_rows);
  p.hs_stride = round32(p.hs_cols);
  p.he_stride = round32(p.he_cols);
  p.ss_stride = round32(p.ss_rows);
  p.n_router = routed_only ? 0 : (E + 1 + p.lg_rows - 1) / p.lg_rows;
  p.n_shup = routed_only ? 0 : (Is + p.hs_cols - 1) / p.hs_cols;
  p.up_jblocks = (I + p.he_cols - 1) / p.he_cols;
  p.n_up = T * k * p.up_jblocks;
  p.n_sd = routed_only ? 0 : (H + p.ss_rows - 1) / p.ss_rows;
  p.down_rows = rows_per_load(I, 4);
  p.n_down = T * (H / p.down_rows);
  return p;
}

struct DecodeArgs {
  int H, E, k, I, Is, T;
  const int8_t* router_q; const uint16_t* router_s;
  const uint8_t* w13_q; const uint16_t* w13_s;
  const uint8_t* w2_q; const uint16_t* w2_s;
  const int8_t* sh13_q; const uint16_t* sh13_s;
  const int8_t* sh2_q; const uint16_t* sh2_s;
  const uint16_t* x;
  uint16_t* out;
  const uint16_t* gain;  // DEC_BLOCK: RMSNorm gain [H] (x is the residual stream)
  float eps;             // DEC_BLOCK: RMSNorm epsilon
  int32_t* ids_out; float* w_out; float* sigma_out;  // nullable
  const int32_t* ids_in; const float* w_in;          // routing given by the caller
  uint32_t* sync;
  float* logits;   // router hand-off:      [n_router][T][lg_stride]
  float* h_s;      // shared gate/up:       [n_shup][T][hs_stride]
  float* h_e;      // expert gate/up:       [n_up][he_stride], he_cols binary16 values each
  float* s_sh;     // shared down:          [n_sd][T][ss_stride]
  DecodePlan p;
};

// floats of each hand-off region
inline size_t decode_region_floats(const DecodePlan& p, int T, int which) {
  switch (which) {
    case 0: return (size_t)p.n_router * T * p.lg_stride;
    case 1: return (size_t)p.n_shup * T * p.hs_stride;
    case 2: return (size_t)p.n_up * p.he_stride;
    default: return (size_t)p.n_sd * T * p.ss_stride;
  }
}

int decode_blocks_per_cu(int mode, bool real_widths, size_t lds_bytes);
int launch_decode(const DecodeArgs& a, int mode, int grid, size_t lds_bytes, hipStream_t s);
bool decode_real_widths(int H, int I, int Is);

}  // namespace moe
