// C ABI: argument validation, workspace layout, path choice and launches.
//
// Everything a call could refuse is checked before the first HIP call, so a
// refused call enqueues nothing and can be exercised without a GPU.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string.h>

#include "chunk.hpp"
#include "decode.hpp"
#include "moe_w4a16.h"

// Scratch of moe_forward_noalloc.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is ever passed to kernels.  Static storage is zero-filled when
// the code object is loaded, so the counters start at zero.
static __device__ __attribute__((aligned(256))) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace moe;

constexpr int kMaxT = 65536;
constexpr int kMaxWidth = 4096;
constexpr size_t kDecodeMaxLds = 64 * 1024;
constexpr uint32_t kPathMask = 0xFFu;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool width_ok(int v) {
  if (v < 64 || v > kMaxWidth) return false;
  if (v % 2048 == 0) return true;
  if (v % 64) return false;
  const int m = v / 64;
  return (m & (m - 1)) == 0;
}

int check_dims(const moe_dims* d, int32_t T) {
  if (!d) return MOE_ERR_NULL;
  if (d->group != kGroup) return MOE_ERR_SHAPE;
  if (d->num_experts < 1 || d->num_experts > kMaxExperts) return MOE_ERR_SHAPE;
  if (d->top_k < 1 || d->top_k > kMaxTopK || d->top_k > d->num_experts) return MOE_ERR_SHAPE;
  if (!width_ok(d->hidden) || !width_ok(d->expert_inter) || !width_ok(d->shared_inter)) return MOE_ERR_SHAPE;
  if ((d->flags & kPathMask) > MOE_PATH_CHUNK ||
      (d->flags & ~(kPathMask | MOE_DEBUG_WAIT_GIVE_UP | MOE_FMT_AFFINE4 | MOE_NORM_GAIN_PLUS_ONE)))
    return MOE_ERR_SHAPE;
  if (T < 0 || T > kMaxT) return MOE_ERR_SHAPE;
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// the few-token path's plan for a grid of nb workgroups (the workspace and
// LDS sizes do not depend on nb)
DecodePlan plan_of(const moe_dims* d, int T, int nb = kGroups * kMaxGroupWgs) {
  return decode_plan(d->hidden, d->num_experts, d->top_k, d->expert_inter, d->shared_inter, T, nb);
}

bool decode_admissible(const moe_dims* d, int T) {
  return T >= 1 && T <= kDecMaxT && decode_lds_bytes(plan_of(d, T)) <= kDecodeMaxLds;
}

bool use_decode(const moe_dims* d, int T) {
  if ((d->flags & kPathMask) == MOE_PATH_CHUNK) return false;
  return decode_admissible(d, T);  // AUTO and DECODE both take it when it fits
}

// each expert with c > 0 rows takes ceil(c / kTileRows) tiles
int max_route_tiles(const moe_dims* d, int T) {
  const int P = T * d->top_k;
  return std::min(d->num_experts, P) + P / kTileRows + 1;
}

// --------------------------------------------------------------- workspace

struct Carve {
  char* base;
  size_t off = 0;
  template <typename P>
  P* take(size_t bytes) {
    P* p = base ? reinterpret_cast<P*>(base + off) : nullptr;
    off = align_up(off + bytes, 256);
    return p;
  }
};

struct DecodeWs {
  uint32_t* sync;
  uint64_t* tagged;
};

// L: sub-blocks per call (each has its own tagged zones)
DecodeWs carve_decode(const moe_dims* d, int T, Carve& c, int L = 1) {
  const DecodePlan p = plan_of(d, T);
  DecodeWs w;
  w.sync = c.take<uint32_t>(kSyncBytes);
  w.tagged = c.take<uint64_t>(p.z_words * 8 * (size_t)L);
  return w;
}

void carve_chunk(const moe_dims* d, int T, Carve& c, ChunkArgs& a) {
  const size_t P = (size_t)T * d->top_k;
  // counters (zero between calls): the last slot is the chunk path's
  uint32_t* sync = c.take<uint32_t>(kSyncBytes);
  a.route_done = sync ? sync + (kCounterPages * kFlagPage - kSyncStride) : nullptr;
  a.logits = c.take<float>((size_t)T * (d->num_experts + 1) * 4);
  a.logits_hi = c.take<float>((size_t)T * (d->num_experts + 1) * 4);
  a.ids = c.take<int32_t>(P * 4);
  a.wts = c.take<float>(P * 4);
  a.sigma = c.take<float>((size_t)T * 4);
  a.wg_cnt = c.take<int32_t>((size_t)d->num_experts * ((T + 15) / 16) * 4);
  a.exp_cnt = c.take<int32_t>((size_t)d->num_experts * 4);
  a.exp_off = c.take<int32_t>((size_t)d->num_experts * 4);
  a.sorted_pair = c.take<int32_t>(P * 4);
  a.sorted_wt = c.take<float>(P * 4);
  a.tiles = c.take<int4>((size_t)(max_route_tiles(d, T) + (T + kSharedRows - 1) / kSharedRows) * 16);
  a.n_tiles = c.take<int32_t>(4);
  a.h = c.take<_Float16>(P * d->expert_inter * 2);
  a.hs = c.take<_Float16>((size_t)T * d->shared_inter * 2);
  a.y = c.take<_Float16>(P * d->hidden * 2);
  a.ys = c.take<_Float16>((size_t)T * d->hidden * 2);
  a.xn = c.take<uint16_t>((size_t)T * d->hidden * 2);
}

size_t workspace_bytes(const moe_dims* d, int T) {
  if (T == 0) return 0;
  Carve c{nullptr};
  ChunkArgs a{};
  carve_chunk(d, T, c, a);
  size_t bytes = c.off;
  if (decode_admissible(d, T)) {
    Carve c2{nullptr};
    carve_decode(d, T, c2);
    bytes = std::max(bytes, c2.off);
  }
  return bytes;
}

// moe_layers_forward: the few-token path's zones for L layers, or the
// grouped-GEMM path's workspace followed by one [T][H] binary16 buffer (the
// output of every other layer)
size_t layers_workspace_bytes(const moe_dims* d, int T, int L) {
  if (T == 0) return 0;
  Carve c{nullptr};
  ChunkArgs a{};
  carve_chunk(d, T, c, a);
  c.take<uint16_t>((size_t)T * d->hidden * 2);
  size_t bytes = c.off;
  if (decode_admissible(d, T)) {
    Carve c2{nullptr};
    carve_decode(d, T, c2, L);
    bytes = std::max(bytes, c2.off);
  }
  return bytes;
}

// --------------------------------------------------------------- device

struct DeviceInfo {
  bool checked = false;
  bool ok = false;
  int cus = 0;
  void* scratch = nullptr;  // this device's address of the static scratch array
  int occ[kDecModes][2][kDecVariants][17] = {};  // blocks per CU by mode, width specialisation, instance
                                                 // and LDS (4 KiB steps)
};

std::mutex g_dev_mu;
DeviceInfo g_dev[64];

int device_info(DeviceInfo** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& di = g_dev[dev];
  if (!di.checked) {
    di.checked = true;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess && strncmp(prop.gcnArchName, "gfx950", 6) == 0) {
      di.ok = true;
      di.cus = prop.multiProcessorCount;
      for (int m = 0; m < kDecModes; ++m)
        for (int r = 0; r < 2; ++r)
          for (int v = 0; v < kDecVariants; ++v)
            for (int s = 0; s <= 16; ++s) di.occ[m][r][v][s] = decode_blocks_per_cu(m, r == 1, v, (size_t)s * 4096);
    }
  }
  if (!di.ok) return MOE_ERR_DEVICE;
  *out = &di;
  return MOE_OK;
}

// --------------------------------------------------------------- static scratch

int scratch_of_current_device(void** out) {
  DeviceInfo* di = nullptr;
  int st = device_info(&di);
  if (st != MOE_OK) return st;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (!di->scratch) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();  // leave no sticky error for the caller's next HIP call
      return MOE_ERR_DEVICE;
    }
    di->scratch = p;
  }
  *out = di->scratch;
  return MOE_OK;
}

// --------------------------------------------------------------- launches

void fill_weights(const moe_weights* w, int8_t const** rq, uint16_t const** rs, uint8_t const** w13q,
                  uint16_t const** w13s, uint8_t const** w2q, uint16_t const** w2s, int8_t const** s13q,
                  uint16_t const** s13s, int8_t const** s2q, uint16_t const** s2s) {
  *rq = w->router_q; *rs = w->router_s; *w13q = w->w13_q; *w13s = w->w13_s; *w2q = w->w2_q; *w2s = w->w2_s;
  *s13q = w->sh13_q; *s13s = w->sh13_s; *s2q = w->sh2_q; *s2s = w->sh2_s;
}

int run_decode(const moe_dims* d, const moe_weights* w, const uint16_t* x, int T, uint16_t* out, int mode,
               int32_t* ids_out, float* w_out, float* sig_out, const int32_t* ids_in, const float* w_in, void* ws,
               hipStream_t s, const uint16_t* gain = nullptr, float eps = 0.f, int L = 1, long long lstride = 0) {
  DeviceInfo* di = nullptr;
  int st = device_info(&di);
  if (st != MOE_OK) return st;
  DecodeArgs a{};
  fill_weights(w, &a.router_q, &a.router_s, &a.w13_q, &a.w13_s, &a.w2_q, &a.w2_s, &a.sh13_q, &a.sh13_s, &a.sh2_q,
               &a.sh2_s);
  a.x = x; a.out = out;
  a.gain = gain; a.eps = eps;
  a.gain_add = (d->flags & MOE_NORM_GAIN_PLUS_ONE) ? 1.0f : 0.0f;
  a.ids_out = ids_out; a.w_out = w_out; a.sigma_out = sig_out;
  a.ids_in = ids_in; a.w_in = w_in;
  a.give_up = (d->flags & MOE_DEBUG_WAIT_GIVE_UP) ? 1 : 0;
  a.affine = (d->flags & MOE_FMT_AFFINE4) ? 1 : 0;
  a.w13_b = w->w13_b; a.w2_b = w->w2_b;
  a.L = L; a.lstride = lstride;
  Carve c{static_cast<char*>(ws)};
  DecodeWs dw = carve_decode(d, T, c, L);
  a.sync = dw.sync; a.tagged = dw.tagged;
  const size_t lds = decode_lds_bytes(plan_of(d, T));
  const int variant = decode_variant(T, a.affine != 0), step = (int)((lds + 4095) / 4096);
  // Every workgroup must be resident at once (they wait for each other, with
  // bounded waits): the grid is what an idle device holds, in whole groups of
  // 8, at most 8 x kMaxGroupWgs; a group needs at least H / 64 members (its
  // members' output rows fit the per-block row buffer).  The instances built
  // for the real widths cover the router rows and shared columns only with
  // kMaxGroupWgs members per group; with fewer the generic instance runs.
  bool real = decode_real_widths(d->hidden, d->expert_inter, d->shared_inter);
  int nj = std::min(kMaxGroupWgs, di->occ[mode][real ? 1 : 0][variant][step] * di->cus / kGroups);
  if (real && nj < kMaxGroupWgs) {
    real = false;
    nj = std::min(kMaxGroupWgs, di->occ[mode][0][variant][step] * di->cus / kGroups);
  }
  if (nj < 1 || nj * kMaxGroupWgs < d->hidden) return MOE_ERR_LAUNCH;
  a.p = plan_of(d, T, kGroups * nj);
  return launch_decode(a, mode, real, lds, s);
}

ChunkArgs chunk_args(const moe_dims* d, const moe_weights* w, const uint16_t* x, int T, uint16_t* out, void* ws) {
  ChunkArgs a{};
  a.H = d->hidden; a.E = d->num_experts; a.k = d->top_k; a.I = d->expert_inter; a.Is = d->shared_inter; a.T = T;
  fill_weights(w, &a.router_q, &a.router_s, &a.w13_q, &a.w13_s, &a.w2_q, &a.w2_s, &a.sh13_q, &a.sh13_s, &a.sh2_q,
               &a.sh2_s);
  a.x = x; a.xa = x; a.out = out;
  a.affine = (d->flags & MOE_FMT_AFFINE4) ? 1 : 0;
  a.w13_b = w->w13_b; a.w2_b = w->w2_b;
  Carve c{static_cast<char*>(ws)};
  carve_chunk(d, T, c, a);
  a.max_route_tiles = max_route_tiles(d, T);
  return a;
}

int check_common(const moe_dims* d, const void* x, int32_t T, void* ws, size_t ws_bytes) {
  int st = check_dims(d, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !ws) return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(ws, 256)) return MOE_ERR_ALIGN;
  if (ws_bytes < workspace_bytes(d, T)) return MOE_ERR_WORKSPACE;
  if ((d->flags & kPathMask) == MOE_PATH_DECODE && !decode_admissible(d, T)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// MOE_FMT_AFFINE4: the routed experts' offset arrays are required and aligned
int check_affine(const moe_dims* d, const moe_weights* w) {
  if (!(d->flags & MOE_FMT_AFFINE4)) return MOE_OK;
  if (!w->w13_b || !w->w2_b) return MOE_ERR_NULL;
  if (!aligned(w->w13_b, 16) || !aligned(w->w2_b, 16)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

bool all16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!aligned(p, 16)) return false;
  return true;
}
bool all4(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && !aligned(p, 4)) return false;
  return true;
}
bool any_null(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p) return true;
  return false;
}

int validate_forward(const moe_dims* dims, const moe_weights* w, const uint16_t* x, int32_t T, const uint16_t* out,
                     const int32_t* ids, const float* weights, const float* shared_gate, const void* ws,
                     size_t ws_bytes);
int launch_forward(const moe_dims* dims, const moe_weights* w, const uint16_t* x, int32_t T, uint16_t* out,
                   int32_t* ids, float* weights, float* shared_gate, void* ws, hipStream_t stream);

}  // namespace

extern "C" {

MOE_API size_t moe_workspace_bytes(const moe_dims* dims, int32_t T) {
  if (check_dims(dims, T) != MOE_OK) return 0;
  return workspace_bytes(dims, T);
}

MOE_API const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "dims or token count outside the admitted shapes";
    case MOE_ERR_ALIGN: return "a pointer is not aligned as required";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_bytes()";
    case MOE_ERR_LAUNCH: return "the HIP runtime refused a kernel launch";
    case MOE_ERR_DEVICE: return "the current device is not gfx950 or cannot be queried";
    case MOE_ERR_SCRATCH: return "the call needs more scratch than moe_forward_noalloc's static array holds";
    default: return "unknown status";
  }
}

MOE_API int moe_route(const moe_dims* dims, const moe_weights* w, const uint16_t* x, int32_t T, int32_t* ids,
                      float* weights, float* shared_gate, float* logits, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  int st = check_common(dims, x, T, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  if (!w) return MOE_ERR_NULL;
  if (any_null({w->router_q, w->router_s, ids, weights})) return MOE_ERR_NULL;
  if (!all16({w->router_q, w->router_s}) || !all4({ids, weights, shared_gate, logits})) return MOE_ERR_ALIGN;
  DeviceInfo* di = nullptr;
  if ((st = device_info(&di)) != MOE_OK) return st;
  ChunkArgs a = chunk_args(dims, w, x, T, nullptr, ws);
  a.ids = ids;
  a.wts = weights;
  if (shared_gate) a.sigma = shared_gate;
  if (logits) a.logits = logits;
  return launch_route_chunk(a, stream);
}

MOE_API int moe_experts_w4a16(const moe_dims* dims, const moe_weights* w, const uint16_t* x, int32_t T,
                              const int32_t* ids, const float* weights, uint16_t* out, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  int st = check_common(dims, x, T, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  if (!w) return MOE_ERR_NULL;
  if (any_null({w->w13_q, w->w13_s, w->w2_q, w->w2_s, ids, weights, out})) return MOE_ERR_NULL;
  if (!all16({w->w13_q, w->w13_s, w->w2_q, w->w2_s, out}) || !all4({ids, weights})) return MOE_ERR_ALIGN;
  if ((st = check_affine(dims, w)) != MOE_OK) return st;
  if (use_decode(dims, T))
    return run_decode(dims, w, x, T, out, DEC_EXPERTS, nullptr, nullptr, nullptr, ids, weights, ws, stream);
  DeviceInfo* di = nullptr;
  if ((st = device_info(&di)) != MOE_OK) return st;
  ChunkArgs a = chunk_args(dims, w, x, T, out, ws);
  a.ids = const_cast<int32_t*>(ids);
  a.wts = const_cast<float*>(weights);
  a.shared_tiles = 0;
  a.cus = di->cus;
  a.ys = nullptr;
  return launch_experts_chunk(a, stream);
}

MOE_API int moe_forward(const moe_dims* dims, const moe_weights* w, const uint16_t* x, int32_t T, uint16_t* out,
                        int32_t* ids, float* weights, float* shared_gate, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  int st = validate_forward(dims, w, x, T, out, ids, weights, shared_gate, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  return launch_forward(dims, w, x, T, out, ids, weights, shared_gate, ws, stream);
}

MOE_API int moe_forward_noalloc(const moe_dims* dims, const moe_weights* w, const uint16_t* x, int32_t T,
                                uint16_t* out, int32_t* ids, float* weights, float* shared_gate,
                                hipStream_t stream) {
  int st = check_dims(dims, T);
  if (st != MOE_OK || T == 0) return st;
  if (workspace_bytes(dims, T) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  // every other check of moe_forward, against an aligned stand-in address for
  // the scratch (validation never dereferences the workspace)
  st = validate_forward(dims, w, x, T, out, ids, weights, shared_gate, reinterpret_cast<void*>(uintptr_t{256}),
                        MOE_NOALLOC_SCRATCH_BYTES);
  if (st != MOE_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != MOE_OK) return st;
  return launch_forward(dims, w, x, T, out, ids, weights, shared_gate, ws, stream);
}

}  // extern "C"

namespace {

int validate_forward(const moe_dims* dims, const moe_weights* w, const uint16_t* x, int32_t T, const uint16_t* out,
                     const int32_t* ids, const float* weights, const float* shared_gate, const void* ws,
                     size_t ws_bytes) {
  int st = check_common(dims, x, T, const_cast<void*>(ws), ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  if (!w) return MOE_ERR_NULL;
  if (any_null({w->router_q, w->router_s, w->w13_q, w->w13_s, w->w2_q, w->w2_s, w->sh13_q, w->sh13_s, w->sh2_q,
                w->sh2_s, out}))
    return MOE_ERR_NULL;
  if (!all16({w->router_q, w->router_s, w->w13_q, w->w13_s, w->w2_q, w->w2_s, w->sh13_q, w->sh13_s, w->sh2_q,
              w->sh2_s, out}) ||
      !all4({ids, weights, shared_gate}))
    return MOE_ERR_ALIGN;
  return check_affine(dims, w);
}

// the complete block on validated arguments
int launch_forward(const moe_dims* dims, const moe_weights* w, const uint16_t* x, int32_t T, uint16_t* out,
                   int32_t* ids, float* weights, float* shared_gate, void* ws, hipStream_t stream) {
  if (use_decode(dims, T))
    return run_decode(dims, w, x, T, out, DEC_FORWARD, ids, weights, shared_gate, nullptr, nullptr, ws, stream);
  DeviceInfo* di = nullptr;
  int st = device_info(&di);
  if (st != MOE_OK) return st;
  ChunkArgs a = chunk_args(dims, w, x, T, out, ws);
  if (ids) a.ids = ids;
  if (weights) a.wts = weights;
  if (shared_gate) a.sigma = shared_gate;
  a.shared_tiles = (T + kSharedRows - 1) / kSharedRows;
  a.cus = di->cus;
  return launch_forward_chunk(a, stream);
}

// the MoE sub-block's checks (every one but the workspace size)
int validate_block(const moe_dims* dims, const moe_weights* w, const uint16_t* h, const uint16_t* gain, float eps,
                   int32_t T, const uint16_t* out, const int32_t* ids, const float* weights, const float* shared_gate,
                   const void* ws) {
  int st = check_dims(dims, T);
  if (st != MOE_OK || T == 0) return st;
  if (!h || !ws || !w) return MOE_ERR_NULL;
  if (any_null({w->router_q, w->router_s, w->w13_q, w->w13_s, w->w2_q, w->w2_s, w->sh13_q, w->sh13_s, w->sh2_q,
                w->sh2_s, out, gain}))
    return MOE_ERR_NULL;
  if (!aligned(h, 16) || !aligned(ws, 256)) return MOE_ERR_ALIGN;
  if (!all16({w->router_q, w->router_s, w->w13_q, w->w13_s, w->w2_q, w->w2_s, w->sh13_q, w->sh13_s, w->sh2_q,
              w->sh2_s, out, gain}) ||
      !all4({ids, weights, shared_gate}))
    return MOE_ERR_ALIGN;
  if ((dims->flags & kPathMask) == MOE_PATH_DECODE && !decode_admissible(dims, T)) return MOE_ERR_SHAPE;
  if ((st = check_affine(dims, w)) != MOE_OK) return st;
  if (!(eps >= 0.f && eps <= 3.0e38f)) return MOE_ERR_SHAPE;  // also refuses NaN and infinity
  const uintptr_t hb = reinterpret_cast<uintptr_t>(h), ob = reinterpret_cast<uintptr_t>(out);
  const uintptr_t n = (uintptr_t)T * dims->hidden * 2;
  if (hb < ob + n && ob < hb + n) return MOE_ERR_SHAPE;  // out overlaps the residual stream
  return MOE_OK;
}

// the sub-block on validated arguments
int launch_block(const moe_dims* dims, const moe_weights* w, const uint16_t* h, const uint16_t* gain, float eps,
                 int32_t T, uint16_t* out, int32_t* ids, float* weights, float* shared_gate, void* ws,
                 hipStream_t stream) {
  if (use_decode(dims, T))
    return run_decode(dims, w, h, T, out, DEC_BLOCK, ids, weights, shared_gate, nullptr, nullptr, ws, stream, gain,
                      eps);
  DeviceInfo* di = nullptr;
  int st = device_info(&di);
  if (st != MOE_OK) return st;
  ChunkArgs a = chunk_args(dims, w, h, T, out, ws);
  if (ids) a.ids = ids;
  if (weights) a.wts = weights;
  if (shared_gate) a.sigma = shared_gate;
  a.gain = gain;
  a.eps = eps;
  a.gain_add = (dims->flags & MOE_NORM_GAIN_PLUS_ONE) ? 1.0f : 0.0f;
  a.xa = a.xn;   // the expert GEMMs read the normalised activations the router GEMM writes
  a.resid = h;   // and the combine adds the residual stream
  a.shared_tiles = (T + kSharedRows - 1) / kSharedRows;
  a.cus = di->cus;
  return launch_forward_chunk(a, stream);
}

template <typename P>
P* offset_ptr(P* p, long long off) {
  return p ? reinterpret_cast<P*>(reinterpret_cast<uintptr_t>(p) + off) : p;
}

// the weights of the layer `off` bytes on from w
moe_weights layer_weights(const moe_weights* w, long long off) {
  moe_weights r = *w;
  r.router_q = offset_ptr(w->router_q, off); r.router_s = offset_ptr(w->router_s, off);
  r.w13_q = offset_ptr(w->w13_q, off); r.w13_s = offset_ptr(w->w13_s, off);
  r.w2_q = offset_ptr(w->w2_q, off); r.w2_s = offset_ptr(w->w2_s, off);
  r.sh13_q = offset_ptr(w->sh13_q, off); r.sh13_s = offset_ptr(w->sh13_s, off);
  r.sh2_q = offset_ptr(w->sh2_q, off); r.sh2_s = offset_ptr(w->sh2_s, off);
  r.w13_b = offset_ptr(w->w13_b, off); r.w2_b = offset_ptr(w->w2_b, off);
  return r;
}

}  // namespace

extern "C" {

MOE_API int moe_block_forward(const moe_dims* dims, const moe_weights* w, const uint16_t* h, const uint16_t* gain,
                              float eps, int32_t T, uint16_t* out, int32_t* ids, float* weights,
                              float* shared_gate, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = validate_block(dims, w, h, gain, eps, T, out, ids, weights, shared_gate, ws);
  if (st != MOE_OK || T == 0) return st;
  if (ws_bytes < workspace_bytes(dims, T)) return MOE_ERR_WORKSPACE;
  return launch_block(dims, w, h, gain, eps, T, out, ids, weights, shared_gate, ws, stream);
}

MOE_API size_t moe_layers_workspace_bytes(const moe_dims* dims, int32_t T, int32_t L) {
  if (check_dims(dims, T) != MOE_OK || L < 1 || L > kMaxLayers) return 0;
  return layers_workspace_bytes(dims, T, L);
}

MOE_API int moe_layers_forward(const moe_dims* dims, const moe_weights* w, const uint16_t* gain, int64_t layer_stride,
                               int32_t L, float eps, const uint16_t* h, int32_t T, uint16_t* out, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  int st = validate_block(dims, w, h, gain, eps, T, out, nullptr, nullptr, nullptr, ws);
  if (st != MOE_OK) return st;
  if (L < 1 || L > kMaxLayers) return MOE_ERR_SHAPE;
  if (layer_stride % 16 != 0) return MOE_ERR_ALIGN;
  if (T == 0) return MOE_OK;
  if (ws_bytes < layers_workspace_bytes(dims, T, L)) return MOE_ERR_WORKSPACE;
  if (use_decode(dims, T))
    return run_decode(dims, w, h, T, out, L > 1 ? DEC_LAYERS : DEC_BLOCK, nullptr, nullptr, nullptr, nullptr, nullptr,
                      ws, stream, gain, eps, L, layer_stride);
  // grouped-GEMM path: one sub-block launch per layer; layer l writes out when
  // L - 1 - l is even and the buffer after the workspace otherwise, so no
  // layer reads and writes the same rows
  Carve c{static_cast<char*>(ws)};
  ChunkArgs scratch{};
  carve_chunk(dims, T, c, scratch);
  uint16_t* buf = c.take<uint16_t>((size_t)T * dims->hidden * 2);
  const uint16_t* in = h;
  for (int l = 0; l < L; ++l) {
    const long long off = layer_stride * l;
    const moe_weights wl = layer_weights(w, off);
    uint16_t* dst = ((L - 1 - l) % 2 == 0) ? out : buf;
    st = launch_block(dims, &wl, in, offset_ptr(gain, off), eps, T, dst, nullptr, nullptr, nullptr, ws, stream);
    if (st != MOE_OK) return st;
    in = dst;
  }
  return MOE_OK;
}

}  // extern "C"
