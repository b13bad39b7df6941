// Arguments and launcher of the few-token (persistent GEMV) path.
#pragma once
#include "common.hpp"

namespace moe {

static constexpr int kDecMaxT = 4;        // tokens per call on this path
static constexpr int kSyncStride = 32;    // counters 128 bytes apart
static constexpr int kSyncBytes = 1024;   // counter region at the start of the workspace
enum { SYNC_ROUTER = 0, SYNC_SHUP = 1, SYNC_UP = 2, SYNC_SD = 3, SYNC_EXIT = 4, SYNC_ERR = 5 };
enum { DEC_FORWARD = 0, DEC_EXPERTS = 1 };

struct DecodeArgs {
  int H, E, k, I, Is, T;
  const int8_t* router_q; const uint16_t* router_s;
  const uint8_t* w13_q; const uint16_t* w13_s;
  const uint8_t* w2_q; const uint16_t* w2_s;
  const int8_t* sh13_q; const uint16_t* sh13_s;
  const int8_t* sh2_q; const uint16_t* sh2_s;
  const uint16_t* x;
  uint16_t* out;
  int32_t* ids_out; float* w_out; float* sigma_out; float* logits_out;  // nullable
  const int32_t* ids_in; const float* w_in;                             // routing given by the caller
  uint32_t* sync;
  float* logits;   // [T][E+1]
  float* h_e;      // [T][k][I]
  float* h_s;      // [T][Is]
  float* s_sh;     // [T][H]
  int n_router, n_shup, n_up, n_sd, n_down;
  int up_jblocks;  // j-blocks per (token, slot)
};

int decode_blocks_per_cu(int mode, size_t lds_bytes);
int launch_decode(const DecodeArgs& a, int mode, int grid, size_t lds_bytes, hipStream_t s);

}  // namespace moe
