// Arguments and launchers of the multi-token (grouped-GEMM) path.
#pragma once
#include "common.hpp"

namespace moe {

static constexpr int kTileRows = 128;  // rows of a routed grouped-GEMM tile (4 MFMA row blocks of 32)
static constexpr int kSharedRows = 64;  // rows of a shared-expert tile (int8 weights need more registers)
static constexpr int kNarrowRows = 16;  // routed tiles of at most this many rows take the narrow path
static constexpr int kNarrowK = 2048;   // ... when K is at most this (the tile's rows stay in LDS)

struct ChunkArgs {
  int H, E, k, I, Is, T;
  const int8_t* router_q; const uint16_t* router_s;
  const uint8_t* w13_q; const uint16_t* w13_s;
  const uint8_t* w2_q; const uint16_t* w2_s;
  const int8_t* sh13_q; const uint16_t* sh13_s;
  const int8_t* sh2_q; const uint16_t* sh2_s;
  const uint16_t* x;   // [T][H] router input (the residual stream in the sub-block)
  const uint16_t* xa;  // [T][H] activations of the expert GEMMs: x, or xn in the sub-block
  uint16_t* out;       // [T][H]
  const uint16_t* gain;  // sub-block: RMSNorm gain [H], or null
  float eps;             // sub-block: RMSNorm epsilon
  float gain_add;        // sub-block: added to every gain element in fp32 (1: the gain holds w of 1 + w)
  uint16_t* xn;          // sub-block: normalised activations [T][H], written by the router GEMM
  const uint16_t* resid; // sub-block: residual added by the combine, or null
  float* logits;       // [T][E+1] (the first K half's partial sums when logits_hi is set)
  float* logits_hi;    // [T][E+1] the second K half's partial sums (router GEMM split over K), or null
  int32_t* ids;        // [T][k]
  float* wts;          // [T][k]
  float* sigma;        // [T]
  int32_t* wg_cnt;     // [E][ceil(T/16)] pairs per top-k workgroup and expert, then their bases (T > 1024)
  int32_t* exp_cnt;    // [E] pairs per expert (T > 1024)
  int32_t* exp_off;    // [E] first place of each expert's run (T > 1024)
  int32_t* sorted_pair;  // [T*k]  pair index at each expert-major position
  float* sorted_wt;    // [T*k]  routing weight of each pair, in the same order
  int4* tiles;         // [max_route_tiles + shared_tiles] (expert or -1 for the shared expert, first
                       // row, rows, 32-row blocks or 0 for a narrow tile), heaviest first
  int32_t* n_tiles;    // tiles written by the bucketing kernel
  _Float16* h;         // [T*k][I]  expert-major rows
  _Float16* hs;        // [T][Is]
  _Float16* y;         // [T*k][H]  weighted expert outputs, row t*k+i for pair (t, i)
  _Float16* ys;        // [T][H]    sigma * shared output, or null (routed half only)
  int shared_tiles;    // number of kSharedRows-token shared-expert tiles (0: routed half only)
  int max_route_tiles; // bound on routed tiles for the grid
  int cus;             // compute units of the device (work pairing in the GEMM kernels)
  uint32_t* route_done;  // counter of finished top-k workgroups (zero between calls)
  int affine;            // routed experts are affine int4 (unsigned codes, w = q s + b)
  const uint16_t* w13_b; const uint16_t* w2_b;  // affine: per-group binary16 offsets
};

int launch_route_chunk(const ChunkArgs& a, hipStream_t s);
int launch_experts_chunk(const ChunkArgs& a, hipStream_t s);
int launch_forward_chunk(const ChunkArgs& a, hipStream_t s);

}  // namespace moe
