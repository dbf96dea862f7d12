/*
 * bqmoe.h -- C ABI of the MI355X (gfx950) routed-expert MoE layer with
 * block-quantized experts.
 *
 * The layer (MiMo-V2.6-Flash-RL shape: every token is routed to 8 of 256
 * experts and the layer has no shared expert -- TrevorJS GGUF card,
 * "Architecture notes"; hidden 4096, expert intermediate 2048) computes for every token t
 *
 *   l      = x_t . Wr^T                    fp32 router (F32 router: savrn
 *                                          card, "Quantization targets")
 *   idx    = top-k experts by l (ties to the lower index)
 *   w      = softmax over the k selected logits
 *   out[t] = sum_s w[s] * D_e (silu(G_e x_t) * (U_e x_t)),  e = idx[s]
 *
 * with fp32 accumulation throughout (expert intermediates exceed fp16's 65504:
 * TrevorJS card, "Recipe", and benthecarman EXL3 card, "Bitrate").
 *
 * Every entry point returns an int status (MOE_OK or a negative code); no C++
 * exception crosses this boundary.  Pointers marked "device" are HIP device
 * addresses (for example torch tensors' data_ptr()); "host" pointers are
 * ordinary memory.  The library never allocates or frees device memory: the
 * caller owns x, router_w, packed_experts, out and the workspace.
 */
#ifndef BQMOE_H
#define BQMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_layer moe_layer; /* opaque handle */

enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,       /* bad argument: null/misaligned pointer, size out of range */
    MOE_EUNSUPPORTED = -2, /* shape or format this build does not implement */
    MOE_EWORKSPACE = -3,   /* workspace missing or smaller than moe_workspace_size */
    MOE_EHIP = -4          /* a HIP launch or runtime call failed */
};

/* Packed expert formats.
 *
 * MOE_FMT_MXFP4 (E2M1 elements, two per byte, one E8M0 exponent per 32
 * consecutive weights of a row -- TrevorJS card, "Architecture notes"):
 *   packed = n_experts experts back to back, each 3*inter*hidden*17/32 bytes:
 *   [gate/up codes][gate/up scales][down codes][down scales].  gate/up is one
 *   matrix of 2*inter rows (rows [0,inter) gate, [inter,2*inter) up) by hidden
 *   columns; down is hidden rows by inter columns.  A matrix of N rows and K
 *   columns is stored as tiles of 16 rows x 32 columns, tile (n/16, k/32) at
 *   index (n/16)*(K/32) + k/32; a tile is 256 code bytes (tile row r at bytes
 *   16r..16r+15, column c in byte c/2, even c in the low nibble) and, in the
 *   scale region, 16 bytes (one E8M0 per tile row).  Weight =
 *   E2M1(code) * 2^(scale-127).  This build supports scale bytes 1..254.
 *
 * MOE_FMT_VQ13R8 (8-dim vector codes: a 13-bit index -- 12-bit stream plus a
 * 1-bit plane -- into a per-layer book, an 8-bit index into a 256-entry
 * residual book, and an F16 gain per row -- Baekpica VQ card, "Recipe"):
 *   packed = [Cb: 8192 x 8 fp16][Rb: 256 x 8 fp16] then n_experts experts of
 *   3*inter*hidden*21/64 + 2*(2*inter + hidden) bytes:
 *   [gu code12][gu plane][gu res][gu gain][dn code12][dn plane][dn res][dn gain].
 *   Tiles are 16 rows x 256 columns (512 vectors); vector (tile row r, vector
 *   column j) is at stream position ((j/8)*16 + r)*8 + j%8 of its tile; code12
 *   is a little-endian 12-bit stream, plane a little-endian bit stream (bit 12
 *   of the index), res one byte per vector; gains are one fp16 per row.
 *   Weight w[n][8v+d] = gain[n] * (Cb[i13][d] + Rb[i8][d]); every sum
 *   Cb[i][d] + Rb[j][d] must be finite in fp16 (|sum| <= 65504).
 *
 * MOE_FMT_VQ13 (the 13-bit stage alone -- Baekpica VQ card, "Recipe": every
 * layer carries it and 32 layers add the residual stage on top, leaving the
 * 13-bit stage's bytes as they are): packed = [Cb: 8192 x 8 fp16] then
 * n_experts experts of 3*inter*hidden*13/64 + 2*(2*inter + hidden) bytes:
 *   [gu code12][gu plane][gu gain][dn code12][dn plane][dn gain],
 * each region as in MOE_FMT_VQ13R8; weight w[n][8v+d] = gain[n] * Cb[i13][d].
 */
enum { MOE_FMT_MXFP4 = 1, MOE_FMT_VQ13R8 = 2, MOE_FMT_VQ13 = 3 };

/* Path selection: AUTO uses the weight-streaming decode kernels for batches of
 * at most MOE_DECODE_MAX_TOKENS tokens (MXFP4) or of one token (VQ13R8,
 * VQ13) and the grouped-GEMM prefill kernels above that; DECODE and PREFILL
 * force one of them (DECODE with a larger T returns MOE_EINVAL).  The decode
 * kernels exist for MXFP4 layers with hidden/256 and inter powers of two
 * (inter <= 2048) and for VQ layers with hidden/256 a power of two up to 16
 * and inter one of 256, 512, 1024, 2048: other layers run the grouped-GEMM
 * kernels at every batch size, and forcing DECODE on them returns
 * MOE_EUNSUPPORTED.
 *
 * Numerics of the grouped-GEMM kernels: MXFP4 gate/up weights are exact in
 * bf16; MXFP4 down weights enter in fp16 as E2M1 * 2^(e - b), b the largest
 * exponent of their 16-row group (exact while a group's exponents span at
 * most 13, beyond that only bits 2^-14 below the group's largest weights are
 * lost); VQ13R8 weights enter as fp16(Cb + Rb) (one rounding, relative
 * error <= 2^-11; VQ13 weights enter as Cb exactly) with the row gain
 * applied in fp32.  The intermediate h of both formats, and x for VQ, enter
 * as fp16 rows scaled by an exact power of two per row (relative error
 * <= 2^-11).  The VQ decode kernels take Cb and
 * Rb unrounded and the activations as above.  All products accumulate in
 * fp32.  The grouped path keeps each route's down output as fp16 times a power
 * of two per 16 (MXFP4) or 4 (VQ) output rows (relative error <= 2^-11) and
 * widens it exactly before the fp32 weighted combine; the decode kernels
 * combine in fp32. */
enum { MOE_PATH_AUTO = 0, MOE_PATH_DECODE = 1, MOE_PATH_PREFILL = 2 };
#define MOE_DECODE_MAX_TOKENS 16

/* Routing weights over a token's k selected experts (the selection itself is
 * the same top-k of the logits either way):
 *   MOE_ROUTE_SOFTMAX  w_s = exp(l_s) / sum_j exp(l_j)
 *   MOE_ROUTE_SIGMOID  w_s = sigma(l_s) / sum_j sigma(l_j), sigma(l) = 1/(1+e^-l)
 * (the TrevorJS card, "Architecture notes", lists sigmoid routing for MiMo;
 * neither form applies an extra scale).  Both are computed in fp32 in a form
 * that stays finite for every finite logit. */
enum { MOE_ROUTE_SOFTMAX = 0, MOE_ROUTE_SIGMOID = 1 };

typedef struct {
    int32_t hidden;     /* H: multiple of 256, at most 8192 */
    int32_t inter;      /* I: multiple of 128 (MXFP4) or 256 (VQ13R8, VQ13) */
    int32_t n_experts;  /* E: 1..256 */
    int32_t top_k;      /* k: 1..8 and k <= E */
    int32_t max_tokens; /* largest T a forward call may pass: 1..65536 */
    int32_t format;     /* MOE_FMT_* */
    int32_t force_path; /* MOE_PATH_* */
    int32_t routing;    /* MOE_ROUTE_* (0, the zero-initialised value, is softmax) */
} moe_layer_desc;

/* Size in bytes of packed_experts for this descriptor (host out-pointer). */
int moe_packed_size(const moe_layer_desc *desc, size_t *bytes);

/* Size in bytes of the device workspace a handle needs (host out-pointer). */
int moe_workspace_size(const moe_layer_desc *desc, size_t *bytes);

/* Validate desc and bind a caller-owned device workspace (256-byte aligned,
 * at least moe_workspace_size bytes, kept alive until moe_layer_destroy).
 * Writes a new handle to *out.  Makes no device call. */
int moe_layer_create(const moe_layer_desc *desc, void *workspace, size_t ws_bytes,
                     moe_layer **out);

/* One forward pass, enqueued on hip_stream (a hipStream_t; NULL = the null
 * stream).  Asynchronous: returns after the last launch, with no host sync.
 *   x_bf16         device, [T][hidden] bfloat16, row-major, 16-byte aligned
 *   T              1..max_tokens
 *   router_w       device, [n_experts][hidden] fp32, row-major, 16-byte aligned
 *   packed_experts device, moe_packed_size bytes in desc->format, 16-byte aligned
 *   out            device, [T][hidden] fp32, row-major, 16-byte aligned;
 *                  fully overwritten
 * The router logit of (t, e) is summed in a fixed order, so routing is
 * reproducible bit for bit: partial c (0..63) accumulates columns k with
 * (k/4) mod 64 == c in ascending k with fused multiply-adds from +0, and the
 * 64 partials are added as a pairwise tree of adjacent blocks.
 * A handle is not reentrant: calls sharing a handle share its workspace and
 * must be ordered (one stream at a time).  Non-finite inputs are outside the
 * contract.  Device faults surface at the caller's next synchronisation. */
int moe_layer_forward(moe_layer *layer, const void *x_bf16, int32_t T, const float *router_w,
                      const void *packed_experts, float *out, void *hip_stream);

/* Copy the routing of the last forward into caller device buffers (any may be
 * NULL to skip), enqueued on hip_stream:
 *   topk_idx [T][k] int32 (slot order: logit descending, index ascending)
 *   topk_w   [T][k] fp32 softmax weights
 *   counts   [n_experts] int32 routes per expert
 *   offsets  [n_experts+1] int32 exclusive prefix sum of counts
 *   perm     [T*k] int32 route ids r = t*k+s sorted by (expert, token)
 *   logits   [T][n_experts] fp32 router logits
 * Returns MOE_EINVAL if no forward has been issued on the handle. */
int moe_layer_routing(moe_layer *layer, int32_t *topk_idx, float *topk_w, int32_t *counts,
                      int32_t *offsets, int32_t *perm, float *logits, void *hip_stream);

/* Path the last forward took (MOE_PATH_DECODE or MOE_PATH_PREFILL), or
 * MOE_EINVAL before the first forward. */
int moe_layer_last_path(const moe_layer *layer);

/* Kernel stages of a forward pass, in launch order. */
enum {
    MOE_STAGE_ROUTER = 0,  /* router logits (plus all of the routing for small batches) */
    MOE_STAGE_SELECT = 1,  /* top-k + softmax (large batches) */
    MOE_STAGE_PERMUTE = 2, /* counting sort of routes by expert (large batches) */
    MOE_STAGE_GATEUP = 3,  /* gate/up projections + SwiGLU */
    MOE_STAGE_DOWN = 4,    /* down projection (plus the combine for small batches) */
    MOE_STAGE_COMBINE = 5, /* weighted combine (large batches) */
    MOE_N_STAGES = 6
};

/* Measurement aid: per-stage kernel timing with HIP events.  slots > 0
 * creates slots sets of event pairs; every later forward records, in the next
 * slot (round robin), one event pair around each kernel it launches, on the
 * forward's stream.  slots == 0 releases the events.  Creating events is a HIP
 * runtime call, so this is not for use under stream capture.  Returns
 * MOE_EINVAL for slots < 0 or > 65536, MOE_EHIP if event creation fails. */
int moe_layer_set_profiling(moe_layer *layer, int32_t slots);

/* Waits for the recorded events and writes elapsed milliseconds to the host
 * array ms[slots][MOE_N_STAGES] (slot order = recording order modulo slots;
 * -1 where a stage did not run).  slots must equal the value given to
 * moe_layer_set_profiling. */
int moe_layer_profile_read(moe_layer *layer, float *ms, int32_t slots);

/* Measurement aid: enqueue the kernels of one stage (MOE_STAGE_*) of the
 * last forward `reps` times back to back on hip_stream, with that forward's
 * inputs, so that events around the call time the stage's kernels alone.
 * Repetition i reads the layer at packed_experts + (i % n_copies) *
 * copy_stride (cycling through copies keeps the weights from being served by
 * the last-level cache); x_bf16, router_w and out are the last forward's
 * arguments (same alignment rules as moe_layer_forward).  Every stage
 * recomputes exactly what the forward computed, so replaying a stage leaves
 * the workspace and out as the forward left them.  Returns MOE_EINVAL before
 * the first forward, for a stage the last forward's path does not run,
 * reps < 1, n_copies < 1, a copy_stride not a multiple of 16, or a bad
 * pointer; MOE_EHIP if a launch fails. */
int moe_layer_replay_stage(moe_layer *layer, int32_t stage, int32_t reps, const void *x_bf16,
                           const float *router_w, const void *packed_experts, size_t copy_stride,
                           int32_t n_copies, float *out, void *hip_stream);

/* Measurement aid: the attainable read bandwidth that the weight-streaming
 * kernels' HBM rates are compared with.  Enqueues `reps` streaming reads of
 * `bytes` of device memory on hip_stream, read i at buf + (i % n_copies) *
 * copy_stride (cycling copies keeps the last-level cache from serving them),
 * each a plain read with 16-byte loads over the whole GPU that writes
 * nothing (sink: a device uint32, written only with vanishing probability,
 * so that the loads are kept).  bytes and copy_stride are multiples of 16,
 * buf 16-byte aligned, copy_stride >= bytes when n_copies > 1.  Returns
 * MOE_EINVAL on a bad argument, MOE_EHIP if a launch fails. */
int moe_read_probe(const void *buf, size_t bytes, size_t copy_stride, int32_t n_copies,
                   int32_t reps, uint32_t *sink, void *hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the forward
 * pass of moe_layer_forward with no handle and no caller workspace.  The
 * workspace is a library-owned device array of MOE_NOALLOC_SCRATCH_BYTES on
 * each GPU the library runs on, held until the process ends; the first call
 * on a device looks its address up (with that device current).
 *   desc   host; validated as by moe_layer_create; max_tokens bounds T and
 *          force_path/routing apply as for a handle
 *   other arguments as for moe_layer_forward (device pointers, same layouts
 *   and alignment; out fully overwritten), enqueued on hip_stream
 * Returns MOE_EINVAL for a bad descriptor or argument, MOE_EWORKSPACE when
 * the workspace of T tokens (moe_workspace_size with max_tokens = T) exceeds
 * the array (at the MiMo shape: up to 96 tokens MXFP4, 91 VQ), MOE_EHIP when the address
 * lookup or a launch fails.  Makes no allocation of any kind.  All calls on
 * one GPU share its array, and a call leaves its contents behind (no kernel
 * reads workspace contents that the same call did not write first): calls
 * that overlap in time on one GPU -- on different streams or from different
 * threads -- race and give undefined results, so order them on one stream. */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)
int moe_forward_noalloc(const moe_layer_desc *desc, const void *x_bf16, int32_t T,
                        const float *router_w, const void *packed_experts, float *out,
                        void *hip_stream);

/* Release the handle (not the workspace).  NULL is a no-op. */
void moe_layer_destroy(moe_layer *layer);

/* Static description of a status code. */
const char *moe_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* BQMOE_H */
