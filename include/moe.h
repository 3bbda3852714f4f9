/*
 * moe.h -- C ABI of the MI355X (gfx950) quantized mixture-of-experts FFN layer.
 *
 * The layer computes, for T tokens x[t] (bf16, hidden size H):
 *   z[t, e]  = Wr[e, :] . x[t] + b[e]                router logits, fp32
 *   S_t      = the k largest z[t, :]                 top-k, ties to the lower expert id
 *   w[t, j]  = softmax over the k selected logits    routing weights
 *   y[t]     = sum_{e in S_t} w[t, e] * W_d[e] (silu(W_g[e] x[t]) * (W_u[e] x[t]))
 * with W_g, W_u, W_d held per expert in one of three precision tiers (bf16,
 * int8 per-channel, int4 group-128), activations in bf16 and all accumulation
 * in fp32.
 *
 * Sources of the operations (web pages):
 *   "Every Expert Counts: ExactMoE for Memory-Efficient W4A16 Inference"
 *     §3.1  router equation z = W_r h and S = TopK(z, k); the router stays BF16;
 *           W_g, W_u, W_d replaced by quantized forms whose dequantized values
 *           define the operation;
 *     §3.2  symmetric group-128 int4 quantizer s = max|W|/7,
 *           q = clip(round(W/s), -8, 7), and the memory equation
 *           P (4/8 + 16/(128*8)) bytes;
 *     §3.3  packed gate/up weights, packed down weights and their FP16 scales
 *           stored once in the kernel's own format;
 *     §3.4  tokens grouped by expert, one fused gate/up grouped GEMM and one
 *           down grouped GEMM per call, a global expert map, router weights
 *           not renormalized, output = sum of the experts' contributions.
 *   "Dynamic Expert Quantization for Scalable Mixture-of-Experts Inference"
 *     (abstract): hot experts at higher precision, low-precision fallback for
 *     the rest, switched through stable expert handles so a forward pass always
 *     runs on a fully materialized expert version.
 *   MxMoE (abstract): GEMMs of different precisions executed together in one
 *     grouped kernel.
 *
 * Conventions for every entry point:
 *   - Return value: MOE_OK (0) or a positive moe_status code.  On error a
 *     message is kept per thread and returned by moe_last_error().
 *   - All argument validation happens on the host before any HIP call; a
 *     rejected call enqueues nothing.
 *   - "device" pointers are HIP device memory (hipMalloc / torch CUDA tensors);
 *     "host" pointers are ordinary CPU memory.  The caller owns every buffer it
 *     passes and keeps it alive until the stream work that uses it completes.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).
 *     moe_route and moe_layer_forward only enqueue work: they never allocate,
 *     never synchronize and never copy data to the host.  Device faults show up
 *     at the caller's next synchronization.
 *   - bf16 tensors are passed as uint16_t bit patterns, row-major.
 *   - Results are deterministic: the same inputs give the same bytes.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = 1,  /* null or misaligned pointer, bad enum value            */
  MOE_ESHAPE = 2,  /* dimension constraint violated                        */
  MOE_ERANGE = 3,  /* non-finite weight or fp16 scale overflow when packing  */
  MOE_ENOSPC = 4,  /* destination or workspace too small                    */
  MOE_EHIP = 5     /* HIP runtime or launch error (text in moe_last_error)  */
} moe_status;

/* Precision tier of one expert. */
typedef enum moe_tier {
  MOE_TIER_BF16 = 0,  /* bf16 weights as given                               */
  MOE_TIER_INT8 = 1,  /* symmetric int8, one fp16 scale per output row         */
  MOE_TIER_INT4 = 2   /* symmetric int4, one fp16 scale per (row, 128 inputs)  */
} moe_tier;

/* How a routing call without logits output computes its top k (the result
 * is the same bit for bit; see moe_route). */
typedef enum moe_router_mode {
  MOE_ROUTER_AUTO = 0,       /* MFMA router when T*E*H is large (default)      */
  MOE_ROUTER_CANONICAL = 1,  /* always the fixed-order fp32 logits kernel      */
  MOE_ROUTER_MFMA = 2        /* MFMA router whenever the call allows it        */
} moe_router_mode;

/* Row order of a packed matrix. */
typedef enum moe_layout {
  MOE_LAYOUT_PLAIN = 0,   /* down projection W_d [H, I]                        */
  MOE_LAYOUT_GATE_UP = 1  /* fused [W_g; W_u] of shape [2I, H], gate rows first;
                             packed with gate and up rows interleaved in blocks
                             of 32 so one tile holds matching gate/up columns  */
} moe_layout;

typedef enum moe_dtype { MOE_DTYPE_BF16 = 0, MOE_DTYPE_F32 = 1 } moe_dtype;

/* One expert's current materialized version (the DynaExq stable handle).
 * w13 is the packed MOE_LAYOUT_GATE_UP blob of [W_g; W_u] ([2I, H]);
 * w2 is the packed MOE_LAYOUT_PLAIN blob of W_d ([H, I]); both device pointers,
 * 256-byte aligned, in the tier given, owned by the caller and kept alive while
 * any forward that can see this handle is in flight.  flags must be 0. */
typedef struct moe_expert_handle {
  int32_t tier;
  int32_t flags;
  const void* w13;
  const void* w2;
} moe_expert_handle;

/* Layer geometry.  Constraints: hidden % 256 == 0, inter % 128 == 0,
 * 1 <= n_experts <= 1024, 1 <= top_k <= min(n_experts, 16), and an expert's
 * bf16 gate/up matrix (2 * inter * hidden * 2 bytes) below 4 GiB. */
typedef struct moe_layer_desc {
  int32_t hidden;     /* H */
  int32_t inter;      /* I (per-expert intermediate size) */
  int32_t n_experts;  /* E */
  int32_t top_k;      /* k */
} moe_layer_desc;

typedef struct moe_layer_s* moe_layer_t;

/* Bytes of a packed blob for an [n_out, k_in] matrix in the given tier,
 * rounded up to a multiple of 256.  int4: n*k/2 + 2*n*k/128 (exactly the
 * ExactMoE §3.2 memory equation); int8: n*k + 2*n; bf16: 2*n*k.
 * Returns 0 for a bad tier or a shape the layout cannot hold
 * (k_in % 128 != 0 or n_out % 64 != 0). */
size_t moe_packed_size(int tier, int64_t n_out, int64_t k_in);

/* Read a packed blob back into row-major codes and scales, on the host (no
 * GPU work; the inverse of the layout moe_quantize_pack writes).  ExactMoE
 * §3.3: packed gate/up codes, packed down codes and FP16 scales in the
 * kernel's own format; this makes that format checkable against the §3.2
 * quantizer without a GPU.
 *   src, src_bytes  host copy of the blob (at least the payload:
 *                   moe_packed_size without its padding).
 *   layout          the layout it was packed with; rows come back in source
 *                   order (gate rows 0..I-1, then up rows, for MOE_LAYOUT_GATE_UP).
 *   q    host int8 [n_out, k_in]: the codes q (int4: -8..7, int8: -128..127);
 *        unused (may be NULL) for MOE_TIER_BF16.
 *   aux  host uint16: int4 the fp16 scale bits [n_out, k_in/128]; int8 the fp16
 *        row scales [n_out]; bf16 the weights' bf16 bits [n_out, k_in].
 * MOE_EINVAL for a bad tier, layout or null pointer, MOE_ESHAPE for a shape the
 * layout cannot hold, MOE_ENOSPC if src_bytes is below the payload. */
int moe_unpack_codes(int tier, int layout, const void* src, size_t src_bytes, int64_t n_out,
                     int64_t k_in, int8_t* q, uint16_t* aux);

/* Quantize (ExactMoE §3.2; int8: the same rule per row with range +-127) and
 * pack one matrix into the kernel's layout, on the GPU.
 *   w_bf16    device, [n_out, k_in] bf16 master weight (PyTorch Linear layout).
 *   layout    MOE_LAYOUT_PLAIN or MOE_LAYOUT_GATE_UP (then n_out = 2I and
 *             rows 0..I-1 are the gate, I..2I-1 the up projection).
 *   n_out % 64 == 0, k_in % 128 == 0, 2 * n_out * k_in < 4 GiB (MOE_ESHAPE).
 *   dst       device, 256-byte aligned, dst_bytes >= moe_packed_size(...).
 * Scales are fp16 (nearest-even of the fp32 quotient max/7 or max/127); codes
 * use round-half-to-even of w / scale.  This is set-up work, not the hot path:
 * it synchronizes the stream and returns MOE_ERANGE if a weight is non-finite
 * or a scale overflows fp16 (dst is then unspecified).  It allocates and frees
 * one 4-byte device flag per call. */
int moe_quantize_pack(int tier, int layout, const uint16_t* w_bf16, int64_t n_out,
                      int64_t k_in, void* dst, size_t dst_bytes, void* stream);

/* Stream-ordered quantize and pack (same operation, arguments and layout as
 * moe_quantize_pack) for repacking while forwards run: it only enqueues work on
 * `stream` (no allocation, no synchronization).  status: device int32, written
 * 0 when the pack starts and nonzero when it ends if a weight is non-finite or a
 * scale overflows fp16 (dst is then unspecified); read it after the stream
 * work completes. */
int moe_quantize_pack_async(int tier, int layout, const uint16_t* w_bf16, int64_t n_out,
                            int64_t k_in, void* dst, size_t dst_bytes, int32_t* status,
                            void* stream);

/* Create a layer.  table: host array of n_experts handles, copied into a
 * library-owned device table on `stream` (stream-ordered).  The layer object
 * is owned by the caller until moe_layer_destroy. */
int moe_layer_create(const moe_layer_desc* desc, const moe_expert_handle* table,
                     void* stream, moe_layer_t* out);

/* Replace handles [first, first+count) (DynaExq-style promotion/demotion).
 * The update is enqueued on `stream`: forwards enqueued on that stream later
 * see the new versions, earlier ones the old.  The host array may be reused as
 * soon as the call returns (handles travel as kernel arguments). */
int moe_layer_set_experts(moe_layer_t layer, int32_t first, int32_t count,
                          const moe_expert_handle* handles, void* stream);

/* Wave execution (ExactMoE §3.4, grouped complete-expert execution; Fig. 1):
 * when the active experts do not all fit in the resident cache of C slots,
 * the layer runs in waves, each over the complete token matrix with an
 * explicit map from global expert ids to resident slots in which every other
 * expert maps to an inactive sentinel, and the wave outputs are accumulated.
 *
 * moe_layer_set_slots: put handles into resident slots [first, first+count)
 * (slot indices 0 .. n_experts-1; handles as for moe_layer_create, validated on
 * the host, stream-ordered like moe_layer_set_experts; the host array may be
 * reused on return).
 *
 * moe_layer_set_slot_map: install the global-expert-to-slot map.
 *   expert_to_slot  host int32 [n_experts]: slot of expert e, or -1 (the
 *                   inactive sentinel).  Every slot it names must have been
 *                   given a handle by moe_layer_set_slots (MOE_EINVAL).
 * Stream-ordered; the host array may be reused on return.  A new layer maps
 * every expert to the sentinel. */
int moe_layer_set_slots(moe_layer_t layer, int32_t first, int32_t count,
                        const moe_expert_handle* handles, void* stream);
int moe_layer_set_slot_map(moe_layer_t layer, const int32_t* expert_to_slot, void* stream);

/* DynaExq (abstract): each expert's usage is estimated from the routing over
 * time; the experts kept at high precision are the most used ones that fit a
 * memory budget; version changes go through stable handles
 * (moe_layer_set_experts) so every forward runs on fully materialized experts.
 *
 * moe_layer_set_hotness: from the next call on, every moe_layer_forward (and
 * every moe_layer_forward_wave with accumulate = 0, i.e. once per layer call)
 * updates hot[e] = decay * hot[e] + (routes to expert e in that call), on the
 * call's stream, in its grouping kernel.  hot: caller-owned device float
 * [n_experts], initialized by the caller; NULL turns the update off.
 * decay in [0, 1] (1: plain counts). */
int moe_layer_set_hotness(moe_layer_t layer, float* hot, float decay);

/* Budget-feasible top-n tier plan (host only, no GPU work).
 *   hot             host float [n_experts]: hotness (no NaN).
 *   bytes_per_tier  host size_t [3]: bytes of one expert (gate/up + down
 *                   blobs) in tier 0 (bf16), 1 (int8), 2 (int4).
 *   budget_bytes    bytes the layer's experts may occupy.
 * Experts are ranked by hotness (descending, ties to the lower id); the n
 * hottest get hi_tier and the rest lo_tier, n the largest value with
 * n * bytes[hi] + (n_experts - n) * bytes[lo] <= budget_bytes.
 * tiers_out: host int32 [n_experts]; n_hi_out (may be NULL) receives n.
 * MOE_ENOSPC if even all experts at lo_tier exceed the budget. */
int moe_plan_tiers(const float* hot, int32_t n_experts, const size_t* bytes_per_tier,
                   size_t budget_bytes, int32_t hi_tier, int32_t lo_tier, int32_t* tiers_out,
                   int32_t* n_hi_out);

/* Router choice of later route and forward calls (moe_router_mode).  The
 * MFMA router needs workspace of its own: size the workspace after setting
 * the mode.  A forward on the decode GEMMs that takes the MFMA router also
 * runs one small pass over x for the GEMMs' group sums (the fixed-order
 * kernel produces them on the way). */
int moe_layer_set_router_mode(moe_layer_t layer, int32_t mode);

/* Free the layer's device state.  The caller must have synchronized every
 * stream that has work using the layer. */
int moe_layer_destroy(moe_layer_t layer);

/* Which grouped-GEMM family and M-tile height each GEMM of a forward of T
 * tokens takes (a diagnostic for callers and tests).
 *   path       gate/up GEMM: 1, few routes per expert (weight streaming, exact
 *              integer MFMA operands); 2, many routes per expert (fp16 MFMA,
 *              dequantized weights rounded once to fp16).
 *   tile_rows  routes per M-tile of the gate/up GEMM: an expert's routes, in
 *              grouped order, are cut into tiles of this many (the last one
 *              ragged).
 *   down_path, down_tile_rows  the same for the down GEMM (either may be
 *              NULL).  The two differ in one case: tens of routes per expert
 *              on layers with many experts, where a path-2 gate/up GEMM feeds
 *              a path-1 down GEMM.
 * Host only; MOE_EINVAL for null path or tile_rows, MOE_ESHAPE for T outside
 * [0, 2^24]. */
int moe_layer_plan(moe_layer_t layer, int32_t T, int32_t* path, int32_t* tile_rows,
                   int32_t* down_path, int32_t* down_tile_rows);

/* Bytes of device workspace a route or forward call with T tokens needs.
 * The workspace is scratch: no state is kept in it between calls, except that
 * a moe_layer_forward_wave with accumulate = 1 reads the routing left by the
 * preceding wave of the same layer call. */
size_t moe_workspace_size(moe_layer_t layer, int32_t T);

/* Routing only (ExactMoE §3.1 and §3.4 grouping).  All pointers device.
 *   x [T, H] bf16;  wr [E, H] bf16;  bias [E] fp32 or NULL.
 *   topk_ids [T, k] int32: the k selected experts of each token, ascending.
 *   topk_w   [T, k] fp32: their softmax weights (aligned with topk_ids).
 *   logits   [T, E] fp32 or NULL: z, summed in the fixed order
 *            chain j = sum over slabs i, then r = 0..7, of x[256i+8j+r]*wr[..]
 *            (32 chains), folded pairwise (j += j+s for s = 16,8,4,2,1), plus b.
 *   expert_offsets [E+1] int32 (4-byte aligned): exclusive prefix sum of
 *                  routes per expert.
 *   sorted_routes  [T*k] int32: route ids r = t*k + j grouped by expert, each
 *                  group in increasing token order.
 *   route_pos      [T*k] int32: position of route r in sorted_routes.
 *   ws: device workspace of ws_bytes >= moe_workspace_size(layer, T).
 * With logits NULL the call may take the MFMA router (moe_layer_set_router_mode;
 * by default when T >= 256, E >= 32 and T*E*H >= 2^29): approximate logits on
 * bf16 MFMA and an error bound against this fixed order leave a few candidate
 * experts per token, whose logits are then summed in the fixed order; the
 * results are the same bit for bit.  With logits NULL, T <= 64, E <= 128 and
 * at most 256 KiB of router weights, one launch computes each token's
 * logits in this fixed order on chip and takes its top k there (again the
 * same results).
 * x and wr must be 16-byte aligned, ws 256-byte aligned.
 * T may be 0 (then only expert_offsets is written, all zero, by a kernel:
 * the call records no memset, so it can be captured in a HIP graph). */
int moe_route(moe_layer_t layer, const uint16_t* x, const uint16_t* wr,
              const float* bias, int32_t T, int32_t* topk_ids, float* topk_w,
              float* logits, int32_t* expert_offsets, int32_t* sorted_routes,
              int32_t* route_pos, void* ws, size_t ws_bytes, void* stream);

/* The whole layer: route, group, gate/up GEMM + SwiGLU, down GEMM, combine.
 *   x [T, H] bf16, wr [E, H] bf16, bias [E] fp32 or NULL (device).
 *   y [T, H] device, bf16 (y_dtype MOE_DTYPE_BF16) or fp32 (MOE_DTYPE_F32);
 *     the bf16 output is the round-to-nearest-even of the fp32 one.
 *   ws: device workspace of ws_bytes >= moe_workspace_size(layer, T), 256-byte
 *     aligned.  x and y must be 16-byte aligned.
 * T may be 0 (nothing is enqueued).  Calls that share a workspace must be
 * ordered on one stream.
 * When either GEMM takes the many-routes-per-expert path (moe_layer_plan path
 * 2), T*H*2 and T*k*I*2 must each stay below 4 GiB (its kernels address these
 * 16-bit activation arrays with 32-bit offsets): MOE_ESHAPE otherwise, before
 * any work is enqueued; split such a batch into several calls. */
int moe_layer_forward(moe_layer_t layer, const uint16_t* x, const uint16_t* wr,
                      const float* bias, int32_t T, void* y, int y_dtype, void* ws,
                      size_t ws_bytes, void* stream);

/* Allocation-free variant of moe_layer_forward, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same computation, arguments and results
 * as moe_layer_forward (bit for bit), but the workspace is a scratch array of
 * MOE_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on,
 * from the first call there until the process ends; the call itself allocates
 * nothing and frees nothing.
 *   MOE_ENOSPC when moe_workspace_size(layer, T) exceeds the scratch (e.g.
 *   above about 800 tokens of a Qwen3-30B-A3B-shaped layer); nothing is
 *   enqueued then.
 * Every call on one GPU uses that GPU's one scratch array: calls that may
 * overlap on one GPU (other streams, other threads, other layers) race and
 * must be ordered by the caller, e.g. on a single stream.  The scratch keeps
 * the last call's contents; no call relies on them. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_layer_forward_noalloc(moe_layer_t layer, const uint16_t* x, const uint16_t* wr,
                              const float* bias, int32_t T, void* y, int y_dtype, void* stream);

/* One wave: as moe_layer_forward, with the router and top-k over all experts
 * unchanged (weights not renormalized within a wave), but only the experts the
 * current slot map sends to a slot contribute, each computed from its slot's
 * handle; every other route contributes nothing.
 *   accumulate = 0: the first wave of a layer call: routes the tokens and
 *                   sets y = the wave's output.
 *   accumulate = 1: a later wave of the same call: keeps the routing (top-k
 *                   ids, weights and activation sums) that the preceding wave
 *                   left in ws, regroups it for the current slot map and adds
 *                   the wave's output to y (y_dtype must be MOE_DTYPE_F32).
 *                   x, wr, bias, T and ws must be those of that first wave,
 *                   ordered after it on the same stream.
 * Over waves whose slot maps partition the experts, the accumulated y is the
 * layer output up to fp32 rounding of the sum order.  Same pointer and
 * stream rules as moe_layer_forward. */
int moe_layer_forward_wave(moe_layer_t layer, const uint16_t* x, const uint16_t* wr,
                           const float* bias, int32_t T, void* y, int y_dtype, int accumulate,
                           void* ws, size_t ws_bytes, void* stream);

/* Optional timing hook: when events (hipEvent_t passed as void*) are set, each
 * forward records events[i] before stage i and events[n-1] after the last
 * stage, on the forward's stream.  Stages: 0 route logits, 1 top-k,
 * 2 grouping, 3 gate/up GEMM + SwiGLU, 4 down GEMM, 5 combine; n = 7.  With
 * n = 9, events[7] and events[8] also receive the gate/up GEMM kernel's own
 * start and end timestamps (hipExtLaunchKernelGGL), without the dispatch gaps
 * a stage boundary includes.  Pass n = 0 to turn it off.  The events are owned
 * by the caller. */
int moe_layer_set_stage_events(moe_layer_t layer, void* const* events, int32_t n);

/* Text of a status code (static storage). */
const char* moe_strerror(int status);

/* Message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/* MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
