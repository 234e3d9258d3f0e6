/*
 * qs_moe.h -- C ABI of the decode-time routed-expert MoE step over 2-bit
 * block-quantised weights, for AMD Instinct MI355X (gfx950).
 *
 * The step: router logits -> top-k with renormalised softmax -> grouping of
 * (token, slot) pairs by expert -> for each selected expert a fused
 * dequantise + gate/up GEMV + SwiGLU -> down GEMV -> weighted combine, plus an
 * ungated high-precision shared expert.  Only the routed experts are 2-bit:
 * gate/up in a codebook 2-bit type, down in a Q2_K type; the router stays
 * fp32 and the shared expert bf16 or 8-bit (QuarkStar README, "Model
 * Weights"; DwarfStar page, "Model Weights" and "Distributed Inference").
 * Dequantisation is fused into the GEMV, since
 * single-stream decode is bound by reading the weights (Quasar README,
 * "Performance model" and "Design decisions").
 *
 * Pointers: every pointer argument is a plain address.  "device" means GPU
 * memory readable by the handle's device; "host or device" means either
 * (the library copies with hipMemcpyDefault).  No pointer is retained
 * after a call returns, except inside the handle's own allocations.
 *
 * Errors: every entry point returns a qs_status.  Arguments are validated on
 * the host before anything is enqueued; on error nothing has been enqueued
 * unless the status is QS_E_HIP, in which case the outputs of that call are
 * undefined (no partial results are defined).  qs_moe_status_string() names
 * a status.
 *
 * Threading: a handle may be used by one host thread at a time.  Calls on one
 * handle share the handle's scratch memory, so two decode calls on the same
 * handle must be ordered (the same stream, or the caller's events).
 */
#ifndef QS_MOE_H
#define QS_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QS_MOE_ABI_VERSION 5

#if defined(__GNUC__)
#define QS_API __attribute__((visibility("default")))
#else
#define QS_API
#endif

typedef enum {
  QS_OK = 0,
  QS_E_INVAL = -1,        /* bad argument: NULL, size, range, alignment */
  QS_E_NOMEM = -2,        /* a device or host allocation failed */
  QS_E_HIP = -3,          /* a HIP runtime call or kernel launch failed */
  QS_E_STATE = -4,        /* a layer used before it was uploaded */
  QS_E_UNSUPPORTED = -5   /* a valid but unsupported configuration */
} qs_status;

/* Routed-expert block formats (256 weights per block, little endian).
 *
 * QS_FMT_Q2K, 84 bytes (the Q2_K type of the pages' down projections):
 *   [0,16)  scales[16]: sub-block i = weights 16i..16i+15 has
 *           sc = scales[i] & 15 and m = scales[i] >> 4
 *   [16,80) qs[64]: weight j has q = (qs[j/4] >> 2*(j%4)) & 3
 *   [80,82) d (IEEE binary16), [82,84) dmin (binary16)
 *   value w_j = d*sc*q_j - dmin*m, rounded once to fp32.
 *
 * QS_FMT_CB2, 70 bytes (the codebook 2-bit type of the pages' gate/up):
 *   [0,2)   d (binary16)
 *   [2,6)   scales: sub-block i = weights 32i..32i+31 has
 *           s = (byte[2 + i/2] >> 4*(i%2)) & 15
 *   [6,38)  idx[32]: group g = weights 8g..8g+7 uses codebook row idx[g]
 *   [38,70) sign[32]: bit b of sign[g] set => weight 8g+b is negated
 *   value w_j = +/- d*s*C[idx[j/8]][j%8] (exact in fp32), with C the
 *   256 x 8 int8 codebook given to qs_moe_create.
 *
 * QS_FMT_Q4K, 144 bytes (the 4-bit Q4_K type at which the pages keep the
 *   routed experts of the last layers: QuarkStar README, "Model Weights",
 *   the Layers34-39Q4KExperts model; DwarfStar page, "Model Weights", q2
 *   with the last 6 layers at q4):
 *   [0,2)    d (binary16), [2,4) dmin (binary16)
 *   [4,16)   scales[12]: sub-block j = weights 32j..32j+31 has 6-bit sc, m:
 *            j < 4:  sc = scales[j] & 63, m = scales[j+4] & 63
 *            j >= 4: sc = (scales[j+4] & 15) | (scales[j-4] >> 6) << 4,
 *                    m  = (scales[j+4] >> 4) | (scales[j] >> 6) << 4
 *   [16,144) qs[128]: weight 64c + r (c < 4) is the low nibble of
 *            qs[32c + r] for r < 32, the high nibble of qs[32c + r - 32]
 *            otherwise
 *   value w_j = d*sc*q_j - dmin*m, rounded once to fp32.
 *
 * Matrix layout: row-major [rows][cols/256] blocks, rows consecutive.
 * gate/up of one expert are [F][H/256] blocks, down is [H][F/256] blocks;
 * the E experts of a layer are consecutive.
 *
 * Shared-expert formats (shared_format):
 * QS_FMT_BF16: bfloat16 weights, row-major [rows][cols].
 * QS_FMT_Q8, 34 bytes per 32 weights (the 8-bit Q8_0 type at which the pages
 *   keep the tensors they do not take to 2 bits: QuarkStar README, "Model
 *   Weights", the "Q8rest" model; DwarfStar page, "Distributed Inference",
 *   the "Q8Shared" model):
 *   [0,2)   d (binary16)
 *   [2,34)  q[32] int8
 *   value w_j = d*q_j (exact in fp32); row-major [rows][cols/32] blocks. */
typedef enum { QS_FMT_BF16 = 0, QS_FMT_Q2K = 1, QS_FMT_CB2 = 2, QS_FMT_Q8 = 3, QS_FMT_Q4K = 4 } qs_format;

/* qs_moe_decode / qs_moe_route flags */
#define QS_DECODE_RESIDUAL 1u   /* x_{l+1} = x_l + MoE_l(u_l); y gets the last x */
#define QS_DECODE_RMSNORM  2u   /* u_l = x_l / sqrt(mean(x_l^2) + 1e-6) (an RMSNorm
                                   without learned weight, as a pre-norm residual
                                   stream applies before each MoE block); without
                                   this flag u_l = x_l */
#define QS_DECODE_STEER    4u   /* steer each layer's MoE output with the
                                   handle's directions (qs_moe_set_steering) */
#define QS_DECODE_EXCLUSIVE 8u  /* the caller runs no other kernel on the device
                                   during the call: the persistent kernel is
                                   dispatched as an ordinary launch instead of a
                                   cooperative one, which saves the cooperative
                                   launch's serialisation (about 20 us per call
                                   on MI355X).  Same kernel, same results.  If
                                   another kernel does hold compute units, some
                                   workgroups start late, the kernel's bounded
                                   waits give up and qs_moe_sync_status reports
                                   QS_E_HIP */

typedef struct qs_moe qs_moe;   /* opaque, owned by the library */

typedef struct {
  int32_t abi_version;     /* QS_MOE_ABI_VERSION */
  int32_t hidden;          /* H: multiple of 256, 256..16384 */
  int32_t n_experts;       /* E: 1..1024 */
  int32_t top_k;           /* k: 1..min(E, 16) */
  int32_t expert_ffn;      /* F: multiple of 256, 256..16384 */
  int32_t shared_ffn;      /* Fs: 0 (no shared expert) or a multiple of 64 up to 16384 */
  int32_t gate_up_format;  /* QS_FMT_CB2 or QS_FMT_Q2K */
  int32_t down_format;     /* QS_FMT_Q2K (QS_FMT_CB2 down is QS_E_UNSUPPORTED) */
  int32_t n_layers;        /* layers held resident: 1..4096 */
  int32_t max_tokens;      /* largest n_tokens of a decode call: 1..256, and
                              max_tokens * top_k <= 1024 */
  int32_t mfma_min_tokens; /* expert bucket size (tokens routed to one expert in
                              one call) from which the matrix-core (MFMA) items
                              replace the GEMV items; a batch that could reach it
                              runs the batched kernel.  0 = library default:
                              batches of up to 4 tokens run the small-batch
                              kernel (GEMV items only) where it fits; larger
                              batches run the batched kernel with every bucket
                              on the matrix cores, one-token batches on the GEMV
                              items (the measured faster choice on MI355X) */
  int32_t device;          /* HIP device ordinal; -1 = the current device */
  int32_t shared_format;   /* QS_FMT_BF16 or QS_FMT_Q8 (shared expert weights) */
  int32_t tail_layers;     /* 0..n_layers: the last tail_layers resident layers
                              hold their routed experts (gate, up and down) in
                              QS_FMT_Q4K instead of gate_up_format/down_format.
                              Those layers run the small-batch kernel for
                              batches it takes (as the 2-bit layers do) and
                              otherwise the batched kernel's GEMV items (no
                              MFMA items); a decode call over both kinds of
                              layer is two launches */
  /* Routed-expert paging, the MI355X form of running a model whose routed
   * experts exceed device memory (QuarkStar README, "Running Models Larger
   * Than Available Memory": non-routed weights stay resident, a prefix of
   * layers can stay fully resident, the selected routed experts go through
   * a bounded cache filled from a slower tier).  The slower tier here is
   * pinned host memory: a decode call reads an expert that is not in the
   * cache straight from host memory over PCIe, so no call waits for a copy
   * or a host round trip; after the call the cache admits the experts it
   * missed (least-recently-used eviction, copies by the DMA engines), in
   * the background of later calls.  Outputs are bitwise the same as with
   * every layer resident: only where the bytes are read from changes. */
  int32_t expert_paging;   /* 0: every layer resident (the next two fields must
                              be 0); 1: paging on */
  int32_t resident_layers; /* paging: layers [0, resident_layers) keep their
                              routed experts in HBM; the routed experts of the
                              later layers ("paged layers") live in pinned host
                              memory.  0..n_layers */
  int32_t cache_slots;     /* paging: HBM slots of the expert cache, each holding
                              one paged expert's gate, up and down matrices;
                              0..(paged layers * E) */
} qs_moe_config;

/* One layer's weights in the raw block layout above.  Host or device
 * pointers; all are only read during qs_moe_upload. */
typedef struct {
  const float*    router;       /* fp32 [E][H] */
  const float*    router_bias;  /* fp32 [E], or NULL for zeros */
  const void*     gate;         /* [E][F][H/256] blocks of gate_up_format (QS_FMT_Q4K in a tail layer) */
  const void*     up;           /* [E][F][H/256] blocks of gate_up_format (QS_FMT_Q4K in a tail layer) */
  const void*     down;         /* [E][H][F/256] blocks of down_format (QS_FMT_Q4K in a tail layer) */
  const void*     shared_gate;  /* [Fs][H] in shared_format; NULL iff Fs == 0 */
  const void*     shared_up;    /* [Fs][H] in shared_format */
  const void*     shared_down;  /* [H][Fs] in shared_format */
} qs_moe_layer_weights;

/* Create a handle for one model shape (the routed-expert MoE layer of the
 * QuarkStar README, "Model Weights": top-k routed experts in 2-bit types
 * plus an unquantised shared expert and router).  Validates cfg, allocates
 * all device memory for n_layers layers and every scratch buffer a decode
 * call of max_tokens needs, so a decode call allocates nothing.
 * codebook: host int8 [256][8] (required iff either format is QS_FMT_CB2,
 * else ignored, may be NULL).  On success *out owns the allocations; on
 * error *out is NULL and nothing stays allocated.  Validation happens before
 * any HIP call, so an invalid cfg fails without touching the GPU.
 * QS_E_UNSUPPORTED: a valid shape for which the device cannot run the
 * persistent decode kernel at some batch size up to max_tokens (no
 * cooperative launch, or a working set larger than a workgroup's LDS). */
QS_API int qs_moe_create(const qs_moe_config* cfg, const int8_t* codebook, qs_moe** out);

/* Copy one layer's weights into the handle's device memory, re-laying the
 * routed blocks out for the kernels (the dequantised values are unchanged).
 * The weights stay resident in HBM, as the pages keep the whole quantised
 * model resident when it fits (QuarkStar README, "Model Weights" and
 * "Running Models Larger Than Available Memory").
 * A paged layer (expert_paging) keeps its router and shared expert in HBM
 * and its re-laid routed experts in the handle's pinned host memory;
 * re-uploading it drops its experts from the cache.
 * hip_stream: a hipStream_t or NULL for the null stream.  Returns after the
 * copies are complete, so the sources may be freed at once.  Re-uploading a
 * layer replaces it. */
QS_API int qs_moe_upload(qs_moe* h, int layer, const qs_moe_layer_weights* w, void* hip_stream);

/* Decode n_tokens tokens through layers [layer0, layer0 + n_layers): the
 * routed-expert MoE step of each layer -- router, top-k with renormalised
 * softmax, fused dequantise + gate/up GEMV + SwiGLU, down GEMV and weighted
 * combine, plus the shared expert (QuarkStar README, "Model Weights"; with
 * n_tokens > 1 the row-batched decode of several sessions in one model step,
 * QuarkStar README, "Server").
 * x: device fp32 [n_tokens][H]; y: device fp32 [n_tokens][H].
 * u_l is x_l, or RMSNorm(x_l) with QS_DECODE_RMSNORM (router and experts both
 * see u_l).  QS_DECODE_STEER steers each layer's MoE output (see
 * qs_moe_set_steering; QS_E_STATE if no directions are set).
 * Without QS_DECODE_RESIDUAL: n_layers must be 1 and y = MoE(u); x and y
 * must not overlap.  With it: x_{l+1} = x_l + MoE_l(u_l) layer by
 * layer and y receives the final x; y == x (in place) is allowed.
 * x and y must be 16-byte aligned.
 * ids_out: device int32 [n_layers][n_tokens][k] or NULL -- selected experts
 * in rank order (logit descending, ties to the lower index).
 * w_out: device fp32 [n_layers][n_tokens][k] or NULL -- their renormalised
 * softmax weights.  One persistent kernel launch on hip_stream, asynchronous;
 * performs no allocation and no host synchronisation.  With expert_paging a
 * call over paged layers also first enqueues the cache admissions of earlier
 * completed calls (see qs_moe_cache_sync), and afterwards copies its ids to
 * host memory and records an event; it does not wait for either.
 * 1 <= n_tokens <= max_tokens.  Non-finite inputs give non-finite outputs but
 * never an out-of-range expert id.
 * Every wait inside the kernel is bounded: a call whose wait gives up (a
 * fault elsewhere on the device, or a limit set by qs_moe_set_wait_limit)
 * still returns here with QS_OK, since the launch itself succeeded; its
 * outputs are undefined, and qs_moe_sync_status reports it.  As with a
 * failed batched step that invalidates every member (QuarkStar README,
 * "Server"), no output of any call since the last qs_moe_sync_status may be
 * used when that call returns QS_E_HIP. */
QS_API int qs_moe_decode(qs_moe* h, int layer0, int n_layers, const float* x, float* y,
                  int n_tokens, uint32_t flags, int32_t* ids_out, float* w_out,
                  void* hip_stream);

/* qs_moe_decode for callers that cannot allocate device memory at the time
 * of the call (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, kernels and results as
 * qs_moe_decode, but every per-call scratch buffer (synchronisation words,
 * flagged words, logits, activation limbs, partial outputs) lives in one
 * static device array of 12 MiB per device, which the library holds until
 * the process ends; the call allocates nothing and runs no allocating
 * library routine.  QS_E_UNSUPPORTED (nothing enqueued, a message on stderr)
 * when this call's scratch -- sized for n_tokens tokens of the handle's
 * shape -- exceeds that array.  All calls on one device share the array and
 * it keeps the last call's contents: calls that overlap on one device (other
 * streams, other handles, other host threads without ordering) race and
 * give undefined results.  qs_moe_sync_status reports its give-ups too. */
QS_API int qs_moe_decode_static(qs_moe* h, int layer0, int n_layers, const float* x, float* y,
                                int n_tokens, uint32_t flags, int32_t* ids_out, float* w_out,
                                void* hip_stream);

/* Wait for hip_stream, then report whether any decode call on this handle
 * (or a qs_moe_decode_static call on its device) since the last
 * qs_moe_sync_status gave up a bounded wait: QS_E_HIP if so
 * (the outputs of those calls are undefined; the handle's synchronisation
 * words are reset, so the next call runs normally), QS_OK otherwise.
 * Synchronises hip_stream; use it where the caller synchronises anyway. */
QS_API int qs_moe_sync_status(qs_moe* h, void* hip_stream);

/* Polls of every bounded wait inside the decode kernels before it gives up;
 * 0 restores the library default (about 0.1 s for a flagged-word read, a few
 * seconds for a grid barrier).  A tiny limit makes waits give up while the
 * data is still on its way: every workgroup then exits through its normal
 * path and qs_moe_sync_status reports the give-up (tests of the error path).
 * Takes effect from the next decode call.  QS_E_INVAL for polls < 0. */
QS_API int qs_moe_set_wait_limit(qs_moe* h, int32_t polls);

/* Directional steering of the MoE outputs (QuarkStar README, "Steering": the
 * FFN output of a layer is edited with the projection of the DwarfStar
 * engine).  A decode call with QS_DECODE_STEER replaces the MoE output m_l
 * of every layer l it runs (routed combine plus shared expert, before the
 * residual add) by
 *     m_l - scale * d_l * (d_l . m_l)
 * in fp32, d_l the layer's direction.  With unit directions a positive scale
 * removes the component along d_l (scale 1 removes it entirely), a negative
 * one amplifies it.  Routing is unaffected (it reads u_l, not m_l).
 * dirs: host or device fp32 [n_layers][H], one direction per resident layer,
 *   used as given (not normalised); copied into device memory the handle
 *   owns (n_layers * H * 4 bytes, counted by qs_moe_memory_bytes).  NULL
 *   frees the directions; a later QS_DECODE_STEER call then fails with
 *   QS_E_STATE (as it does before the first qs_moe_set_steering).
 * scale: finite, else QS_E_INVAL.
 * Returns after the copy.  Must not overlap a decode call on the handle.
 * The steered combine of the small-batch kernel exchanges one more set of
 * flagged words per layer (the per-workgroup partial dot products); the
 * batched kernel takes one more grid barrier per layer. */
QS_API int qs_moe_set_steering(qs_moe* h, const float* dirs, float scale, void* hip_stream);

/* Expert cache of a handle with expert_paging (QS_E_STATE without it).
 *
 * Policy: least-recently-used over all slots of all paged layers.  The uses
 * of a decode call are the distinct (layer, expert) pairs of its paged
 * layers in (layer, token, rank) order; a use of a cached expert refreshes
 * it, a use of an uncached one admits it into a free slot (lowest index
 * first) or else evicts the least recently used expert.  A call's uses are
 * applied after the call, in call order; qs_moe_decode applies those of
 * earlier calls that have completed by the time it is called, without
 * waiting, so the cache state a call sees may lag by a few calls (outputs
 * never depend on it).  qs_moe_decode_static neither reads back ids nor
 * updates the cache (it reads through the map as it stands).
 *
 * qs_moe_cache_sync: waits for hip_stream and every pending call, applies
 *   their uses and enqueues the admissions on hip_stream, then waits for
 *   them; afterwards the cache state is exactly that of the policy applied
 *   to every completed call in order.
 * qs_moe_cache_preload: the popularity hotlist warm start (QuarkStar README,
 *   "Running Models Larger Than Available Memory": warm streaming preloads a
 *   bounded popularity hotlist).  keys: host int32 [n][2] of (layer,
 *   expert), hottest first; each paged pair not cached takes a free slot
 *   until none is left (nothing is evicted).  Synchronises like
 *   qs_moe_cache_sync.  QS_E_INVAL for a key outside the paged layers.
 * qs_moe_cache_stats: host uint64 out[8] = {hits, misses, admissions,
 *   evictions, preloaded, slots in use, slots, host bytes of the paged
 *   experts}, counted over the uses applied so far.
 * qs_moe_cache_slots: host int32 out[cache_slots][2]: (layer, expert) held by
 *   each slot, (-1, -1) for a free slot, as of the uses applied so far. */
QS_API int qs_moe_cache_sync(qs_moe* h, void* hip_stream);
QS_API int qs_moe_cache_preload(qs_moe* h, const int32_t* keys, int n, void* hip_stream);
QS_API int qs_moe_cache_stats(qs_moe* h, uint64_t* out);
QS_API int qs_moe_cache_slots(qs_moe* h, int32_t* out);

/* Routing only (diagnostics and tests): the router, top-k and grouping steps
 * of one layer for n_tokens tokens, with every intermediate written out
 * (the selection of the QuarkStar README, "Model Weights": the router stays
 * at full precision and picks the top-k routed experts).
 * Any output pointer may be NULL.  All outputs are device memory:
 *   logits_out fp64 [n_tokens][E]       router logits
 *   ids_out    int32 [n_tokens][k]      as in qs_moe_decode
 *   w_out      fp32 [n_tokens][k]       as in qs_moe_decode
 *   group_out  int32 [3*E + 2 + n_tokens*k]:
 *      [0, E)              count of pairs per expert
 *      [E, 2E+1)           exclusive offsets (offsets[E] = n_tokens*k)
 *      [2E+1, 2E+1+T*k)    pairs token*k + slot, ordered by (expert, token)
 *      [2E+1+T*k]          number of experts with a non-empty bucket, U
 *      [2E+2+T*k, 3E+2+T*k) those experts ascending (entries >= U are -1)
 * flags: 0 or QS_DECODE_RMSNORM (routes u = RMSNorm(x) as qs_moe_decode does).
 * Asynchronous on hip_stream. */
QS_API int qs_moe_route(qs_moe* h, int layer, const float* x, int n_tokens, uint32_t flags,
                 double* logits_out, int32_t* ids_out, float* w_out, int32_t* group_out,
                 void* hip_stream);

/* Dequantise one matrix from the handle's device copy with the same field
 * decoding the GEMV kernels use (tests of the IQ2_XXS-class gate/up, Q2_K
 * down, Q4_K and Q8_0 shared types of the QuarkStar README, "Model Weights").
 * which: 0 gate, 1 up, 2 down of routed expert `expert`; 3 gate, 4 up,
 * 5 down of the shared expert (expert ignored; QS_E_INVAL when Fs == 0).
 * out: device fp32 [F][H] (gate/up), [H][F] (down), [Fs][H] (shared
 * gate/up) or [H][Fs] (shared down).  Asynchronous. */
QS_API int qs_moe_dequant(qs_moe* h, int layer, int expert, int which, float* out, void* hip_stream);

/* Bytes of device memory the handle holds (weights + scratch; the paged
 * experts' host copies are not counted, see qs_moe_cache_stats); the pages
 * budget the resident weight footprint against the device memory
 * (QuarkStar README, "Model Weights"). */
QS_API int qs_moe_memory_bytes(const qs_moe* h, uint64_t* bytes);

/* Synchronise the handle's device, then free everything.  NULL is a no-op. */
QS_API int qs_moe_destroy(qs_moe* h);

/* Static string naming a status; never NULL. */
QS_API const char* qs_moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* QS_MOE_H */
