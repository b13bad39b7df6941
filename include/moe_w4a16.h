/*
 * moe_w4a16.h — C ABI of the routed Mixture-of-Experts FFN under W4A16 on
 * AMD MI355X (gfx950).
 *
 * What the library computes (the Chimera notebook "Qwen3.6-35B-A3B Decode on
 * Chimera GPNPU", section 5 "Validate the MoE FFN block"): for every token x,
 *
 *     out = routed(x) + sigmoid(x . W_sg) * shared(x)
 *
 *   - router logits l = x . W_r^T over E experts; the router rows are stored
 *     int8 with binary16 group-64 scales, stacked with the shared-gate row W_sg
 *     as row E (the TensorFold PR "Qwen3.6-35B-A3B on Metal on the routed
 *     path", section "Design");
 *   - softmax over the E logits, keep the top k, renormalise the k kept
 *     probabilities (the Chimera notebook, section 5.2); ties go to the lower
 *     expert index;
 *   - routed(x) = sum_i w_i * FFN_{e_i}(x) with SwiGLU experts
 *     FFN(x) = (silu(x W_gate^T) * (x W_up^T)) W_down^T, int4 weights
 *     (the Chimera notebook, pipeline intro: routed experts int4);
 *   - shared(x) is a dense SwiGLU expert with int8 weights, applied to every
 *     token (same notebook: shared expert int8, activations fp16).
 *
 * Storage format (every weight array is row-major, K-contiguous):
 *   - int4 code: two's-complement nibble in [-8, 7]; element 2j of a row is
 *     the low nibble of byte j, element 2j+1 the high nibble;
 *   - int8 code: two's complement;
 *   - scales: IEEE binary16 bit patterns, one per 64 consecutive K elements of
 *     a row ([rows][K/64]); dequantised weight = code * scale (no zero point).
 *     Every dequantised weight must be a finite binary16 value (|code * scale|
 *     <= 65504).  The few-token path and the router GEMM apply scales in fp32;
 *     the grouped expert GEMMs round each dequantised weight to binary16 before
 *     the matrix core (relative error <= 2^-11, or an absolute error <= 2^-25
 *     for weights under 2^-14 in magnitude, which binary16 holds as subnormals);
 *   - activations x and out: IEEE binary16 [T][H].
 *
 * Conventions for every entry point:
 *   - `dims` and `w` are host pointers to host structs; every array pointer
 *     inside `w` and every other array argument is a DEVICE pointer of the
 *     current HIP device, owned by the caller.  The library never allocates,
 *     frees, copies host<->device or synchronises.
 *   - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *     immediately; results are ready when the stream reaches that point.
 *   - Every argument is validated before anything is enqueued: a call that
 *     returns an error has enqueued nothing and changed nothing.
 *   - T = 0 is a valid no-op (returns MOE_OK, enqueues nothing).
 *   - Alignment: weight arrays, x and out 16 bytes; ids, routing weights,
 *     sigma and logits 4 bytes; the workspace 256 bytes.
 *   - Shape admission: G = 64; 1 <= k <= E <= 256 and k <= 8; each of H, I and
 *     Is is 64 * 2^m or a multiple of 2048, and at most 4096; 0 <= T <= 65536.
 *   - The workspace (`ws`, `ws_bytes` >= moe_workspace_bytes(dims, T)) is
 *     scratch owned by the caller.  Its first 40 KiB hold counters that must
 *     be zero before the first call that uses the workspace (allocate it
 *     zero-filled); every call keeps them consistent for the next one (arrival
 *     counters return to zero, call counters advance by a fixed amount).  The
 *     32-bit word at byte offset 1024 counts the workgroups whose bounded wait
 *     gave up (see below); it is never reset by the library.  Calls that share
 *     a workspace must be ordered (same stream, or synchronised).
 *   - The few-token path (T <= 4) is one launch whose workgroups wait for each
 *     other with bounded waits (about a second each), so it needs the whole
 *     grid resident at once: nothing else may hold the device's compute units
 *     for that long while it runs.  If a wait gives up, the call writes NaN to
 *     the outputs that depend on the missing values (in practice all of out),
 *     counts the give-up in the workspace word above, and leaves the workspace
 *     usable: the next call is unaffected.  MOE_DEBUG_WAIT_GIVE_UP forces this
 *     path for testing.
 *   - Device-side routing ids outside [0, E) passed to moe_experts_w4a16
 *     contribute nothing (they are never dereferenced).
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

/* status codes */
#define MOE_OK 0
#define MOE_ERR_NULL (-1)      /* a required pointer is NULL */
#define MOE_ERR_SHAPE (-2)     /* dims or T outside the admitted shapes */
#define MOE_ERR_ALIGN (-3)     /* a pointer is not aligned as required */
#define MOE_ERR_WORKSPACE (-4) /* ws_bytes < moe_workspace_bytes(dims, T) */
#define MOE_ERR_LAUNCH (-5)    /* the HIP runtime refused a launch */
#define MOE_ERR_DEVICE (-6)    /* the current device is not gfx950 or cannot be queried */
#define MOE_ERR_SCRATCH (-7)   /* moe_forward_noalloc: the call needs more than MOE_NOALLOC_SCRATCH_BYTES */

/* dims.flags: execution path (both compute the same result) */
#define MOE_PATH_AUTO 0u   /* few tokens: persistent GEMV launch; otherwise grouped MFMA GEMMs */
#define MOE_PATH_DECODE 1u /* force the few-token path (T <= 4) */
#define MOE_PATH_CHUNK 2u  /* force the grouped-GEMM path */
/* dims.flags bit (test hook): every bounded wait of the few-token path gives
 * up at once, as it would if the launch's workgroups could not all run at the
 * same time.  The call then writes NaN to out (see the few-token path's
 * failure contract below) and the workspace stays usable. */
#define MOE_DEBUG_WAIT_GIVE_UP 0x100u
/* dims.flags bit: the routed experts are affine int4 (the form of a 4-bit
 * affine checkpoint such as the one the TensorFold PR runs, "Receipts"):
 * codes are UNSIGNED nibbles q in [0, 15] (same packing: element 2j in the
 * low nibble of byte j) and each group of 64 along K has a binary16 scale s
 * (w13_s, w2_s) and a binary16 offset b (w13_b, w2_b):  w = q * s + b.
 * The router and the shared expert keep their symmetric int8 form. */
#define MOE_FMT_AFFINE4 0x200u
/* dims.flags bit for moe_block_forward and moe_layers_forward: `gain` holds w
 * and the norm multiplies by (1 + w), formed in fp32 (the form of the
 * published Qwen3.5-MoE RMSNorm, whose weight is stored as w).  Without it
 * `gain` is the multiplier as applied.  Other entry points ignore it. */
#define MOE_NORM_GAIN_PLUS_ONE 0x400u

typedef struct {
  int32_t hidden;       /* H */
  int32_t num_experts;  /* E */
  int32_t top_k;        /* k */
  int32_t expert_inter; /* I: routed-expert intermediate width */
  int32_t shared_inter; /* Is: shared-expert intermediate width */
  int32_t group;        /* G: quantisation group along K, must be 64 */
  uint32_t flags;       /* MOE_PATH_*, optionally | MOE_FMT_AFFINE4 | MOE_NORM_GAIN_PLUS_ONE | MOE_DEBUG_WAIT_GIVE_UP */
} moe_dims;

typedef struct {
  const int8_t* router_q;   /* [E+1][H] int8; row E is the shared-gate row */
  const uint16_t* router_s; /* [E+1][H/G] binary16 */
  const uint8_t* w13_q;     /* [E][2I][H/2] int4 pairs; rows 0..I-1 gate, I..2I-1 up */
  const uint16_t* w13_s;    /* [E][2I][H/G] */
  const uint8_t* w2_q;      /* [E][H][I/2] int4 pairs (down projection) */
  const uint16_t* w2_s;     /* [E][H][I/G] */
  const int8_t* sh13_q;     /* [2Is][H] int8; rows 0..Is-1 gate, Is..2Is-1 up */
  const uint16_t* sh13_s;   /* [2Is][H/G] */
  const int8_t* sh2_q;      /* [H][Is] int8 */
  const uint16_t* sh2_s;    /* [H][Is/G] */
  const uint16_t* w13_b;    /* MOE_FMT_AFFINE4 only: [E][2I][H/G] binary16 offsets (else NULL, not read) */
  const uint16_t* w2_b;     /* MOE_FMT_AFFINE4 only: [E][H][I/G] binary16 offsets (else NULL, not read) */
} moe_weights;

/* Bytes of workspace a call with these dims and T tokens needs (any entry
 * point).  Returns 0 for inadmissible dims. */
MOE_API size_t moe_workspace_bytes(const moe_dims* dims, int32_t T);

/* Router alone (the Chimera notebook, section 5: the router validated on its
 * own): logits of the E experts and of the shared gate, top-k selection,
 * renormalised weights and the shared-expert gate value.
 *   x            [T][H] binary16
 *   ids          [T][k] int32, experts in descending logit order (ties: lower index)
 *   w            [T][k] float, renormalised weights, same order
 *   shared_gate  [T] float, sigmoid of the shared-gate logit
 *   logits       [T][E+1] float (column E: shared-gate logit), or NULL */
MOE_API int moe_route(const moe_dims* dims, const moe_weights* w, const uint16_t* x, int32_t T, int32_t* ids,
                      float* weights, float* shared_gate, float* logits, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* Routed half alone, with caller-supplied routing (the Chimera notebook,
 * section 5: routed experts without the shared expert):
 *   out[t] = sum_i weights[t][i] * FFN_{ids[t][i]}(x[t])     binary16 [T][H]
 * Ids outside [0, E) contribute nothing.  Router rows and shared-expert
 * arrays in `w` are not read (they may be NULL). */
MOE_API int moe_experts_w4a16(const moe_dims* dims, const moe_weights* w, const uint16_t* x, int32_t T,
                              const int32_t* ids, const float* weights, uint16_t* out, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* The complete block: out = routed + sigmoid(x . W_sg) * shared, binary16
 * [T][H].  ids [T][k], weights [T][k] and shared_gate [T] receive the routing
 * when non-NULL. */
MOE_API int moe_forward(const moe_dims* dims, const moe_weights* w, const uint16_t* x, int32_t T, uint16_t* out,
                        int32_t* ids, float* weights, float* shared_gate, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* The MoE sub-block of a decoder layer (the Chimera notebook, sections 7 and
 * 10: post-attention RMSNorm -> MoE FFN -> residual), fused into the block:
 *   a[t]   = binary16( h[t] / sqrt(mean_j h[t][j]^2 + eps) * gain )
 *   out[t] = binary16( h[t] + moe_forward's block applied to a[t] )
 * with one rounding of out.
 *   h     [T][H] binary16, the residual stream (16-byte aligned; must not alias out)
 *   gain  [H] binary16, the norm's multiplier as applied (16-byte aligned), or
 *         w of a (1 + w) multiplier with MOE_NORM_GAIN_PLUS_ONE
 *   eps   finite, >= 0; anything else is refused with MOE_ERR_SHAPE
 * ids, weights and shared_gate receive the routing of a[t] when non-NULL, as
 * for moe_forward. */
MOE_API int moe_block_forward(const moe_dims* dims, const moe_weights* w, const uint16_t* h, const uint16_t* gain,
                              float eps, int32_t T, uint16_t* out, int32_t* ids, float* weights,
                              float* shared_gate, void* ws, size_t ws_bytes, hipStream_t stream);

/* L MoE sub-blocks applied in turn (the Chimera notebook, "Pipeline": the
 * decoder runs as one kernel per token, every layer's weights a fixed offset
 * from the previous layer's, so the entry takes the same pointers for any
 * depth):
 *   h_0 = h,  h_{l+1} = moe_block_forward(layer l)(h_l)  (binary16 between layers),
 *   out = h_L.
 * Layer l's arrays are those of `w` and `gain` (layer 0) each moved on by
 * l * layer_stride bytes; layer_stride is a multiple of 16 (0: the same weights
 * every layer).  The result equals L moe_block_forward calls chained through
 * binary16 buffers, bit for bit.
 *   L     1 .. 256 (else MOE_ERR_SHAPE)
 *   h     [T][H] binary16, must not alias out; gain as for moe_block_forward
 *   ws    ws_bytes >= moe_layers_workspace_bytes(dims, T, L), with the
 *         workspace rules above
 * With T <= 4 (and MOE_PATH_CHUNK not set) all L layers are one persistent
 * launch: a layer's output reaches the next layer through the workspace and
 * the next layer's router and shared-expert rows are loaded while the current
 * layer's last sums are formed.  Otherwise the layers are L launches in order.
 * No routing outputs. */
MOE_API size_t moe_layers_workspace_bytes(const moe_dims* dims, int32_t T, int32_t L);
MOE_API int moe_layers_forward(const moe_dims* dims, const moe_weights* w, const uint16_t* gain, int64_t layer_stride,
                               int32_t L, float eps, const uint16_t* h, int32_t T, uint16_t* out, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/* moe_forward without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments and
 * result as moe_forward; the scratch memory is a static array of
 * MOE_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU the library
 * runs on, held until the process ends (its address is looked up once per
 * device, on the first call there).  A call whose moe_workspace_bytes(dims, T)
 * exceeds that size is refused with MOE_ERR_SCRATCH before anything is
 * enqueued (at real widths the limit admits up to 159 tokens).  Every call on
 * one GPU shares that GPU's array: calls that may overlap on one GPU (other
 * streams, other threads) race and must be ordered by the caller.  Each
 * completed call leaves the array as the next call needs it (arrival counters
 * zero, call counters advanced). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
MOE_API int moe_forward_noalloc(const moe_dims* dims, const moe_weights* w, const uint16_t* x, int32_t T,
                                uint16_t* out, int32_t* ids, float* weights, float* shared_gate,
                                hipStream_t stream);

/* Static description of a status code. */
MOE_API const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H */
