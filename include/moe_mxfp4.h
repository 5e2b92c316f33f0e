/*
 * moe_mxfp4.h -- C ABI of the MI355X (gfx950) MXFP4 expert-weight MoE decode layer.
 *
 * The layer (the decode-time MoE of "3 Ways to Improve MoE Inference on NVIDIA
 * DGX Spark", digest sections 1-3 and 5): a router scores all E experts of each
 * token and keeps the top-k (8 of 512) with renormalised softmax weights; one
 * shared expert always runs; all (token, expert) pairs are sorted by expert so
 * each expert's MXFP4 weights are read once per batch (MoE-SpeQ article, section
 * 4.2); each expert computes h = SiLU(x Wg^T) * (x Wu^T) and h Wd^T; a weighted
 * cross-expert reduction forms y (MoE-SpeQ article, section 3.2).
 *
 * Conventions shared by every call
 *  - Pointers marked "device" are HIP device pointers owned by the caller; the
 *    library allocates no device memory, never copies device data to the host
 *    and keeps no state between calls (so calls from several host threads are
 *    safe as long as they share no buffer, stream or event).  All work is
 *    enqueued on `stream` (a hipStream_t; NULL = the default stream) and is
 *    asynchronous; no call synchronises.  The _ex calls can also take helper
 *    streams and events from the caller (moe_exec_opts).
 *  - Argument checks run on the host before anything is enqueued and return a
 *    status; nothing is launched when a check fails.  MOE_ERR_HIP means a launch
 *    was rejected by the HIP runtime (e.g. no gfx950 device).  No call aborts,
 *    throws or falls back to another implementation.
 *  - Calls that share a workspace or output buffer on one stream are ordered by
 *    the stream; concurrent calls on different streams must not share them.
 *  - MXFP4 tensor [N][K] (K % 32 == 0), row-major:
 *      codes  uint8 [N][K/2]:  byte j of a row holds element 2j in its low nibble
 *                              and element 2j+1 in its high nibble;
 *      scales uint8 [N][K/32]: E8M0 byte s of block b scales elements 32b..32b+31
 *                              of the row by 2^(s-127).
 *    A 4-bit code c is E2M1: sign = bit 3, magnitude = {0,0.5,1,1.5,2,3,4,6}[c&7].
 *    (The pages name MXFP4 but do not define it; this is the OCP MX v1.0 format.)
 *    Dequantisation is exact for scale bytes in [2, 252]; outside that range
 *    results are undefined (the layer's workloads use [120, 127]).
 *  - Activations are bf16 bit patterns (uint16).  Outputs are float32.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,       /* a required pointer is NULL                              */
  MOE_ERR_SHAPE = 2,      /* a size is outside the documented limits                 */
  MOE_ERR_ALIGN = 3,      /* a pointer is not 16-byte aligned where required          */
  MOE_ERR_WORKSPACE = 4,  /* workspace smaller than moe_workspace_bytes(...)          */
  MOE_ERR_HIP = 5         /* the HIP runtime rejected a launch                       */
} moe_status;

/* Limits checked by every call. */
#define MOE_MAX_EXPERTS 1024   /* E (routed experts)                        */
#define MOE_MAX_TOPK 32        /* k, also k <= E                            */
#define MOE_MAX_HIDDEN 8192    /* H, multiple of 32                         */
#define MOE_MAX_INTER 4096     /* I, multiple of 32                         */
#define MOE_MAX_TOKENS 65536   /* M                                         */
#define MOE_LMHEAD_MAX_TOKENS 8 /* M of moe_lmhead_fp8_logits; also M*H <= 32768 */

/* Expert bank of one layer: E routed experts, then (if has_shared) the shared
 * expert at index E.  All four pointers are device pointers, 16-byte aligned.
 *   w13_q [E+S][2I][H/2], w13_s [E+S][2I][H/32]: rows 0..I-1 are W_gate, rows
 *        I..2I-1 are W_up (each [I][H], reduction over H);
 *   w2_q  [E+S][H][I/2],  w2_s  [E+S][H][I/32]:  W_down [H][I] (reduction over I). */
typedef struct {
  const uint8_t* w13_q;
  const uint8_t* w13_s;
  const uint8_t* w2_q;
  const uint8_t* w2_s;
  int32_t num_experts;  /* E */
  int32_t hidden;       /* H */
  int32_t inter;        /* I */
  int32_t has_shared;   /* S: 0 or 1 */
} moe_mxfp4_weights;

/* Execution options of moe_layer_ex and moe_mxfp4_forward_ex.  Zero-initialise
 * it; every field is optional, and a NULL options pointer means all zeros.
 *   act8            0: bf16 activations into the experts (W4A16, as moe_layer);
 *                   1: the W4A8 variant (as moe_layer_w4a8, see below)
 *   helper_streams  two hipStream_t of the caller (default priority), or both
 *                   NULL.  For batches of more than 4 tokens the few-token and
 *                   scaled-MFMA expert kernels then run on them beside the GEMV
 *                   kernels on `stream`; they are forked from `stream` and joined
 *                   back to it with helper_events, so the call stays ordered on
 *                   `stream` and can be captured into a HIP graph.  NULL: every
 *                   kernel runs on `stream`, in order.  Calls enqueued at the
 *                   same time must not share helper streams or events.
 *   helper_events   four hipEvent_t of the caller (timing may be disabled);
 *                   required when helper_streams are given, else ignored
 *   gateup_events   two hipEvent_t, or NULL: they take the begin and end
 *                   timestamps of the GEMV gate/up kernel (for M <= 4 it
 *                   includes the in-block routing), so hipEventElapsedTime gives
 *                   that kernel's own execution time (for measurement)
 *   down_events     the same for the GEMV down kernel
 * Status: MOE_ERR_SHAPE for act8 outside {0, 1}; MOE_ERR_NULL for one helper
 * stream without the other, or helper streams with a NULL event. */
typedef struct {
  int32_t act8;
  void* helper_streams[2];
  void* helper_events[4];
  void* gateup_events[2];
  void* down_events[2];
} moe_exec_opts;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(moe_status st);

/* Bytes of device workspace moe_mxfp4_forward needs for these sizes
 * (0 if the sizes are outside the limits). */
size_t moe_workspace_bytes(int32_t M, int32_t top_k, int32_t E, int32_t H, int32_t I);

/* Router: logits, top-k and renormalised weights ("NVIDIA three-layer
 * optimisation" news rewrite, paragraph on sparse activation and expert
 * routing; the gate stays in high precision per the MoE-SpeQ article, 2.1).
 *   x            device bf16 [M][H]
 *   w_router     device fp32 [E][H]
 *   logit_bias   device fp32, NULL (no bias), [E] (bias_row_stride = 0) or
 *                [M][E] (bias_row_stride = E); added to the logits before top-k
 *   logits       device fp32 [M][E], output: x . w_router[e] + bias, fp32
 *                accumulation of exact bf16*fp32 products
 *   topk_ids     device int32 [M][k], output: per token the k largest logits in
 *                descending order, ties to the lower expert index
 *   topk_weights device fp32 [M][k], output: exp(l_i - l_max) / sum over the kept
 *                experts (the softmax renormalised over the top-k)
 * Limits: 1 <= M <= MOE_MAX_TOKENS, 32 <= H <= MOE_MAX_HIDDEN, H % 32 == 0,
 * 1 <= k <= min(E, MOE_MAX_TOPK), E <= MOE_MAX_EXPERTS; x and w_router 16-byte aligned. */
moe_status moe_route(const uint16_t* x, const float* w_router, const float* logit_bias,
                     int64_t bias_row_stride, int32_t M, int32_t H, int32_t E, int32_t top_k,
                     float* logits, int32_t* topk_ids, float* topk_weights, void* stream);

/* The top-k + renormalised softmax step of moe_route alone, on given logits
 * (device fp32 [M][E]); outputs as in moe_route.  Same limits on M, E, k. */
moe_status moe_topk_softmax(const float* logits, int32_t M, int32_t E, int32_t top_k,
                            int32_t* topk_ids, float* topk_weights, void* stream);

/* Sort the M*k flattened pairs p = t*k + s by expert, stably (MoE-SpeQ article,
 * section 4.2: collect every token's expert assignments, order them by expert
 * id, run each expert once over its tokens).
 *   topk_ids        device int32 [M][k], values in [0, E)
 *   expert_offsets  device int32 [E+1], output: pairs of expert e occupy
 *                   sorted_pairs[expert_offsets[e] .. expert_offsets[e+1])
 *   sorted_pairs    device int32 [M*k], output: pair indices, ascending within an expert
 *   active_experts  device int32 [E], output: the D experts with at least one
 *                   pair, ascending, in entries 0..D-1 (the rest untouched)
 *   num_active      device int32 [1], output: D
 * Limits as moe_route.  Ids outside [0, E) are skipped (they take no place in the
 * output and expert_offsets[E] counts only the valid ones). */
moe_status moe_sort_by_expert(const int32_t* topk_ids, int32_t M, int32_t top_k, int32_t E,
                              int32_t* expert_offsets, int32_t* sorted_pairs,
                              int32_t* active_experts, int32_t* num_active, void* stream);

/* The experts and the combine (digest "3 Ways to Improve MoE Inference on
 * NVIDIA DGX Spark", sections 2-3: MXFP4 experts plus one shared expert;
 * MoE-SpeQ article, 3.2 and 4.2: each expert runs once over its sorted pairs
 * and the expert outputs are reduced across experts): for every active expert
 * e and each of its pairs p = t*k + s, h = SiLU(x_t Wg_e^T) * (x_t Wu_e^T) and
 *   y_t = sum_s topk_weights[t][s] * (h Wd_e^T) + (shared expert of x_t, weight 1).
 * Reads the sort outputs on the device (num_active is never copied to the host).
 * Arithmetic: MXFP4 weights decode exactly; products accumulate in fp32; h is
 * carried between the projections as two terms (bf16 hi + lo, or two MXFP8
 * terms for experts with >= 16 tokens), about 16 significant bits.
 *   x                      device bf16 [M][H], 16-byte aligned
 *   w                      host pointer to the expert bank descriptor
 *   topk_weights           device fp32 [M][k]
 *   expert_offsets, sorted_pairs, active_experts, num_active: moe_sort_by_expert outputs
 *   y                      device fp32 [M][H], output (overwritten)
 *   workspace              device, >= moe_workspace_bytes(M, k, E, H, I) bytes, 256-byte
 *                          aligned; its contents on entry are ignored
 * Limits as moe_route plus 32 <= I <= MOE_MAX_INTER, I % 32 == 0. */
moe_status moe_mxfp4_forward(const uint16_t* x, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                             const float* topk_weights, const int32_t* expert_offsets,
                             const int32_t* sorted_pairs, const int32_t* active_experts,
                             const int32_t* num_active, float* y, void* workspace,
                             size_t workspace_bytes, void* stream);

/* moe_mxfp4_forward with execution options (helper streams, timing events,
 * W4A8 activations: moe_exec_opts).  opts may be NULL. */
moe_status moe_mxfp4_forward_ex(const uint16_t* x, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                                const float* topk_weights, const int32_t* expert_offsets,
                                const int32_t* sorted_pairs, const int32_t* active_experts,
                                const int32_t* num_active, float* y, void* workspace, size_t workspace_bytes,
                                const moe_exec_opts* opts, void* stream);

/* The whole layer in one call: moe_route, moe_sort_by_expert and
 * moe_mxfp4_forward with the same arguments and outputs, fused into fewer
 * launches.  For M <= 4 (decode, speculative verify) there are three: the
 * router logits, then a gate/up kernel each of whose workgroups takes the
 * top-k and the expert sort itself from the logits, then down.  For M <= 8 the
 * top-k and the sort share one workgroup; above, they are separate launches.
 * Every intermediate output (logits, ids, weights, sort outputs) is still
 * written, with the values the separate calls give.
 * Limits: those of the three calls; x, w_router and the bank 16-byte aligned,
 * workspace 256-byte aligned. */
moe_status moe_layer(const uint16_t* x, const float* w_router, const float* logit_bias,
                     int64_t bias_row_stride, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                     float* logits, int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                     int32_t* sorted_pairs, int32_t* active_experts, int32_t* num_active, float* y,
                     void* workspace, size_t workspace_bytes, void* stream);

/* moe_layer for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same call without the workspace arguments.  Its workspace is a static
 * device array of MOE_NOALLOC_WORKSPACE_BYTES inside the library, one per GPU
 * (held until the process ends), found with hipGetSymbolAddress on the first
 * call on each device; the call allocates nothing.  Every call on a GPU shares
 * that GPU's array, and it keeps the last call's contents (the layer ignores
 * them on entry): calls that overlap on one GPU -- on different streams, or
 * from different host threads -- race and must not be made.
 * Same arguments, outputs and limits as moe_layer, plus:
 * moe_workspace_bytes(M, k, E, H, I) <= MOE_NOALLOC_WORKSPACE_BYTES, else
 * MOE_ERR_WORKSPACE (the Ling layer, H = 2560 and I = 768 with 512 experts
 * top-8, fits up to M = 57). */
#define MOE_NOALLOC_WORKSPACE_BYTES (8u << 20)
moe_status moe_layer_noalloc(const uint16_t* x, const float* w_router, const float* logit_bias,
                             int64_t bias_row_stride, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                             float* logits, int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                             int32_t* sorted_pairs, int32_t* active_experts, int32_t* num_active, float* y,
                             void* stream);

/* moe_layer with execution options (moe_exec_opts: the W4A8 variant, helper
 * streams for batches, timing events of the gate/up and down kernels).  Same
 * arguments, outputs and limits as moe_layer; opts may be NULL (= moe_layer). */
moe_status moe_layer_ex(const uint16_t* x, const float* w_router, const float* logit_bias,
                        int64_t bias_row_stride, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                        float* logits, int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                        int32_t* sorted_pairs, int32_t* active_experts, int32_t* num_active, float* y,
                        void* workspace, size_t workspace_bytes, const moe_exec_opts* opts, void* stream);

/* Measurement hook: the floor for streaming a set of byte ranges on this chip.
 * One kernel reads every range the way the decode kernels stream expert
 * weights -- 16 bytes per lane, each workgroup's chunk of
 * MOE_READ_PROBE_CHUNK bytes requested at once -- and does nothing else; the
 * bench reads a layer's expert weights with it to set their kernels' times
 * against.
 *   addrs       device uint64 [n]: range start addresses, 16-byte aligned
 *   sizes       device int64 [n]: range lengths in bytes, multiples of 16, each
 *               in [16, max_bytes] (ranges are read, never written)
 *   max_bytes   host: the largest size, a multiple of 16
 *   out         device uint32 [n][C], C = ceil(max_bytes / MOE_READ_PROBE_CHUNK):
 *               out[i][c] = XOR of the little-endian 32-bit words of bytes
 *               [c, c + 1) x MOE_READ_PROBE_CHUNK of range i (0 past its end)
 *   out_words   >= n * C
 *   start_event, stop_event  hipEvent_t recorded at the kernel's start and end
 *               (both or neither; NULL: none)
 * MOE_ERR_NULL, MOE_ERR_SHAPE (n outside [1, 65535], bad max_bytes, short
 * out), MOE_ERR_ALIGN (addrs, sizes not 8-byte aligned, out not 4-byte
 * aligned); sizes outside the stated bounds are undefined. */
#define MOE_READ_PROBE_CHUNK 16384
moe_status moe_read_probe(const uint64_t* addrs, const int64_t* sizes, int32_t n, int64_t max_bytes, uint32_t* out,
                          size_t out_words, void* start_event, void* stop_event, void* stream);

/* Measurement hook of the decode path (M <= 4, H = 2560, I = 768): moe_layer
 * with kernel instances that also write phase timestamps (the GPU's 100 MHz
 * constant clock, s_memrealtime) of thread 0 of every workgroup: per
 * workgroup index w = y * gridDim.x + x of each kernel's own grid,
 *   stamps[16w + 0..8]:  gate/up kernel entry, token 0's logits loaded, its
 *                        top-k threshold, its top-k done (two or more
 *                        tokens), the workgroup's routing barrier passed,
 *                        slot known, weight loads issued, first weight block
 *                        used, h written (the routing writer: its outputs
 *                        written);
 *   stamps[16w + 9..13]: down kernel entry, record loaded, loads issued,
 *                        first weight block used, y added.
 * Stamps a workgroup does not reach keep their prior value.  Results are those
 * of moe_layer.
 *   stamps      device uint64 [num_stamps], 8-byte aligned
 *   num_stamps  >= moe_layer_probe_stamps(M, top_k, E, H, I)
 * MOE_ERR_SHAPE for sizes the decode path does not cover (the helper returns 0
 * for them) or a short buffer. */
size_t moe_layer_probe_stamps(int32_t M, int32_t top_k, int32_t E, int32_t H, int32_t I);
moe_status moe_layer_probe(const uint16_t* x, const float* w_router, const float* logit_bias,
                           int64_t bias_row_stride, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                           float* logits, int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                           int32_t* sorted_pairs, int32_t* active_experts, int32_t* num_active, float* y,
                           void* workspace, size_t workspace_bytes, unsigned long long* stamps,
                           size_t num_stamps, void* stream);

/* moe_layer with a hint from a draft pass (speculative decoding predicts the
 * experts of the coming tokens: MoE-SpeQ article, 4.1).  Same arguments,
 * outputs and limits as moe_layer, plus two timing events of the gate/up
 * kernel (as moe_exec_opts.gateup_events; may be NULL) and:
 *   hint_experts device int32 [*num_hint]: the routed experts the draft
 *                predicts for this layer, ascending (e.g. moe_sort_by_expert's
 *                active_experts of the draft's ids); entries outside [0, E)
 *                are ignored
 *   num_hint     device int32 [1]: their count
 * Both NULL: moe_layer.  Only one NULL: MOE_ERR_NULL.  For M <= 4 the
 * gate/up workgroups whose waves are idle during the routing read one word
 * of every 64-byte line of their rows of hint_experts[slot], so a right guess
 * finds the stream in L2; the results never depend on the hint. */
moe_status moe_layer_hinted(const uint16_t* x, const float* w_router, const float* logit_bias,
                            int64_t bias_row_stride, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                            float* logits, int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                            int32_t* sorted_pairs, int32_t* active_experts, int32_t* num_active, float* y,
                            void* workspace, size_t workspace_bytes, const int32_t* hint_experts,
                            const int32_t* num_hint, void* start_event, void* stop_event, void* stream);

/* ------------------------------------------------------------------- W4A8
 * The baseline deployment of the Ling model runs the MXFP4 experts with 8-bit
 * activations, W4A8 (digest, section 2).  Here the 8-bit format is MXFP8 in
 * the OCP microscaling sense (the pages name W4A8 only): blocks of 32
 * consecutive elements along the reduction axis share one E8M0 scale
 * X = 2^(floor(log2 amax) - 8), exponent clamped to [-127, 127] (2^-127 for an
 * all-zero block); each element is the E4M3 code nearest to v / X, ties to
 * even, the quotient clamped to +-448. */

/* Quantise bf16 rows [rows][K] to MXFP8 along K.
 *   x       device bf16 [rows][K], 16-byte aligned
 *   codes   device uint8 [rows][K] E4M3 codes, 16-byte aligned, or NULL
 *   scales  device uint8 [rows][K/32] E8M0 bytes (exponent + 127), or NULL
 *   values  device bf16 [rows][K]: each code's value (code * X), 16-byte aligned,
 *           or NULL; exact for blocks whose largest magnitude is >= 2^-110
 * At least one output. Limits: rows >= 1, K >= 32, K % 32 == 0, rows*K < 2^40. */
moe_status moe_mxfp8_quantize(const uint16_t* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                              uint16_t* values, void* stream);

/* moe_layer in the W4A8 variant.  Same arguments, outputs and limits; the
 * routing (logits, ids, weights, sort outputs) is moe_layer's, on the bf16 x.
 * The experts (routed and shared) take x as MXFP8 (each element replaced by
 * its code's value), and the down projection takes h as MXFP8 along I,
 * quantised from h as computed (fp32 sums, carried between the kernels as two
 * bf16 terms, about 16 significant bits).  Experts with >= 16 tokens run on the scaled MXFP4
 * matrix cores with one MXFP8 activation term. */
moe_status moe_layer_w4a8(const uint16_t* x, const float* w_router, const float* logit_bias,
                          int64_t bias_row_stride, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                          float* logits, int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                          int32_t* sorted_pairs, int32_t* active_experts, int32_t* num_active, float* y,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Dequantise an MXFP4 tensor [rows][cols] (layout above) to fp32 with the same
 * device routine the expert kernels use (exposes it for exact checks).
 *   q device uint8 [rows][cols/2], s device uint8 [rows][cols/32], out device fp32 [rows][cols]
 * Limits: rows >= 1, cols >= 32, cols % 32 == 0, rows*cols < 2^40; q 16-byte aligned. */
moe_status moe_mxfp4_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols,
                                float* out, void* stream);

/* ------------------------------------------------------------ Expert prefetch
 * Speculative decoding can tell ahead of a layer which experts it will use:
 * the draft model's routing for the next tokens is counted into an expert
 * heat map, and the predicted experts are fetched in priority order on a
 * stream of their own before the verify pass needs them (MoE-SpeQ article,
 * 4.1 and 4.3).  Here every layer's experts already reside in HBM, so a
 * prefetch reads the predicted experts' weights into the GPU's memory-side
 * last-level cache (the Infinity Cache), from which the layer's own reads are
 * then served.  Results of the layer do not depend on whether, or what, was
 * prefetched. */
#define MOE_PREFETCH_MAX_DRAFT_IDS 1048575  /* n_ids of moe_prefetch_select      */
#define MOE_PREFETCH_MAX_LIST 65535         /* max_ids of moe_prefetch_experts   */

/* The prefetch list of one layer from the draft's routing.
 *   draft_ids    device int32 [n_ids]: the routed expert ids the draft pass
 *                produced for this layer (e.g. moe_route's topk_ids of the
 *                draft tokens, flattened); ids outside [0, E) count for nothing
 *   expert_ids   device int32 [max_experts], output: the shared expert (index E)
 *                first when has_shared, then every expert with heat > 0 (heat =
 *                how many draft ids equal it) by descending heat, ties to the
 *                lower index, cut to max_experts entries; entries past the list
 *                are set to -1.  (The article's priority 0.6 heat + 0.3 size +
 *                0.1 transfer time orders a bank of equal-sized experts by heat.)
 *   num_selected device int32 [1], output: the list's length
 * Limits: 0 <= n_ids <= MOE_PREFETCH_MAX_DRAFT_IDS, 1 <= E <= MOE_MAX_EXPERTS,
 * has_shared in {0, 1}, 0 <= max_experts <= MOE_PREFETCH_MAX_LIST; pointers
 * 4-byte aligned.  One workgroup. */
moe_status moe_prefetch_select(const int32_t* draft_ids, int32_t n_ids, int32_t E, int32_t has_shared,
                               int32_t max_experts, int32_t* expert_ids, int32_t* num_selected, void* stream);

/* Read the listed experts' weights (every byte of the chosen arrays) so that
 * they are cache-resident when the layer runs.
 *   w          host pointer to the expert bank descriptor (as moe_mxfp4_forward)
 *   expert_ids device int32 [max_ids]: bank entries to read (0..E-1 routed, E the
 *              shared expert when the bank has one); entries outside the bank
 *              are skipped, a repeated entry is read again
 *   num_live   device int32 [1] (e.g. moe_prefetch_select's num_selected): only
 *              entries 0..min(*num_live, max_ids)-1 are read; NULL: all max_ids
 *   parts      1: gate/up codes and scales, 2: down codes and scales, 3: both
 *   checksums  device uint32 [max_ids]: entry r's sum, modulo 2^32, of the
 *              little-endian 32-bit words read is added to checksums[r] (so
 *              every load is used and the bytes read can be checked); skipped
 *              entries add nothing.  The caller sets the initial values.
 * Limits: the bank's sizes as moe_mxfp4_forward, its pointers 16-byte aligned;
 * 0 <= max_ids <= MOE_PREFETCH_MAX_LIST (0 launches nothing); 1 <= parts <= 3;
 * expert_ids, num_live and checksums 4-byte aligned.  Launched as one grid row
 * of 64 KB workgroups per list entry; calls on other streams run beside it. */
moe_status moe_prefetch_experts(const moe_mxfp4_weights* w, const int32_t* expert_ids, const int32_t* num_live,
                                int32_t max_ids, int32_t parts, uint32_t* checksums, void* stream);

/* ---------------------------------------------------------------- FP8 LM head
 * The LM head projects the hidden state onto the vocabulary (2,560 -> 157,184
 * for the Ling model: digest, section 2).  Its bf16 weights are quantised
 * online to FP8, which halves the bytes read per decode step (digest,
 * section 4; Vietnamese rewrite, section 2).  FP8 is OCP E4M3 ("FN": bias 7,
 * no infinities, 0x7F/0xFF NaN, largest finite 448) -- the pages name FP8 only.
 * Weights row-major [V][H]; one fp32 scale per row. */

/* Quantise a bf16 head [V][H] to E4M3 codes [V][H] and fp32 row scales [V]:
 * s[v] = amax(|w[v][:]|) / 448 in fp32 (1 for an all-zero row); codes[v][k] =
 * the E4M3 value nearest to clamp(w[v][k] / s[v], -448, 448) (fp32 quotient),
 * ties to the even mantissa, sign kept (so -0 and negative values that round
 * to zero give 0x80).
 *   w_bf16 device bf16 bits [V][H], 16-byte aligned; codes device uint8 [V][H],
 *   8-byte aligned; scales device fp32 [V].  All caller-owned.
 * Limits: V >= 1, 32 <= H <= MOE_MAX_HIDDEN, H % 32 == 0.  Non-finite weights:
 * undefined. */
moe_status moe_lmhead_fp8_quantize(const uint16_t* w_bf16, int32_t V, int32_t H, uint8_t* codes,
                                   float* scales, void* stream);

/* logits[t][v] = (sum_k x[t][k] * e4m3(codes[v][k])) * scales[v] for M decode
 * tokens (W8A16: x stays bf16; each product is exact in fp32, the sum is fp32,
 * then one multiply by the scale).  Reads each code once per call.
 *   x device bf16 bits [M][H], 16-byte aligned; codes device uint8 [V][H],
 *   16-byte aligned; scales device fp32 [V]; logits device fp32 [M][V],
 *   overwritten.
 * Limits: 1 <= M <= MOE_LMHEAD_MAX_TOKENS, M*H <= 32768, V >= 1,
 * 32 <= H <= MOE_MAX_HIDDEN, H % 32 == 0.  NaN codes (0x7F, 0xFF): undefined. */
moe_status moe_lmhead_fp8_logits(const uint16_t* x, const uint8_t* codes, const float* scales, int32_t M,
                                 int32_t V, int32_t H, float* logits, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
