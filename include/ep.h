/* ep.h -- C ABI of libep.so: MoE expert-parallel dispatch / combine, the
 * token exchange of DeepEP-style expert parallelism, on one MI355X (gfx950).
 *
 * What the calls compute. The DeepEP usage guide (zhouruolin.cn, "DeepEP：MoE
 * 专家并行 EP 通信 kernel 编译与使用指南", section 5 "使用方法") gives the
 * interface this ABI follows: a buffer created once for a maximum number of
 * tokens per rank, hidden size and top-k; dispatch(x, topk_idx,
 * topk_weights, num_experts, ...) returning the received activations, the
 * received top-k weights and a handle; combine(expert_output, handle)
 * returning the combined activations; and combine_backward /
 * dispatch_backward reusing the forward handle. The launch report
 * (czhn.yksolo.com, section on the normal kernels) and the blog.hotdry.top
 * notes (section 5, precision choice) pair FP8 dispatch with BF16 combine.
 * The pages do not define the layout step, the receive layout, the FP8 scale
 * granularity or the combine arithmetic; the readings used here are stated at
 * each call below.
 *
 * Expert-parallel group on one GPU. The R expert-parallel ranks are R
 * disjoint partitions of this GPU's memory: receive rows
 * [d*cap_rows, (d+1)*cap_rows) belong to rank d. Source tokens are split in
 * contiguous blocks of T/R per source rank; expert e lives on rank e/(E/R).
 *
 * Conventions.
 *  - All array arguments are DEVICE pointers to memory the caller owns
 *    (allocated with hipMalloc or by torch); the library never frees them.
 *    Struct arguments (ep_config, ep_layout, ep_handle, ep_sizes) are HOST
 *    structs whose pointer fields are device pointers.
 *  - Every compute call is asynchronous on `stream` (a hipStream_t passed as
 *    void*; NULL = the legacy default stream) and returns once its kernels are
 *    queued. Inputs must stay alive and unmodified until the stream has passed
 *    the call.
 *  - bf16 values are passed as uint16_t bit patterns, FP8 as OCP e4m3fn bytes,
 *    weights and scales as IEEE fp32, routing indices as int32 with -1 meaning
 *    "no expert in this slot". All arrays are row-major and dense.
 *  - A negative return value means nothing was launched (EP_ERR_*).
 *    Data-dependent problems (bad expert ids, capacity overflow) are reported
 *    through sticky device status bits (EP_ST_*, read with ep_get_status); the
 *    kernels never write outside the caller's buffers when one is raised.
 *  - One ep_ctx holds a small device workspace used by the layout kernel;
 *    calls on the same ctx must be ordered on one stream (calls on different
 *    streams that use the same ctx at the same time race). A context belongs
 *    to the device current at ep_create: a call made while another device is
 *    current returns EP_ERR_ARG.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EP_ABI_VERSION 2

/* return codes */
#define EP_OK 0
#define EP_ERR_ARG (-1)   /* invalid config, null pointer, size mismatch, handle from another config */
#define EP_ERR_ALIGN (-2) /* a row array is not 16-byte aligned */
#define EP_ERR_HIP (-3)   /* a HIP runtime call failed */
#define EP_ERR_NOMEM (-4) /* the workspace could not be allocated */
#define EP_ERR_SCRATCH (-5) /* ep_dispatch_with_layout_noalloc: the workload needs more than its static workspace */

/* sticky device status bits */
#define EP_ST_BAD_EXPERT 1u /* an index outside [-1, E): that slot was dropped */
#define EP_ST_DUP_EXPERT 2u /* an expert repeated within a token: repeats after the first were dropped */
#define EP_ST_CAPACITY 4u   /* a rank needs more than cap_rows rows: rows past cap_rows were dropped */
#define EP_ST_TIMEOUT 8u    /* the layout scan gave up waiting for a predecessor tile (results invalid) */
#define EP_ST_BAD_HANDLE 16u /* a handle position outside [-1, R*cap_rows): that slot was skipped */

typedef void *ep_stream_t;
typedef struct ep_ctx ep_ctx;

/* Problem size, fixed when the context is created (the guide's buffer is
 * created for a maximum token count, hidden size and top-k).
 * Limits: 0 <= num_tokens <= 2^24, num_tokens % num_ranks == 0;
 * 1 <= num_topk <= 32; 1 <= num_ranks <= 64; 1 <= num_experts <= 1024,
 * num_experts % num_ranks == 0; 8 <= hidden <= 65536, hidden % 8 == 0
 * (hidden % 128 == 0 for FP8 dispatch); 0 <= cap_rows,
 * num_ranks * cap_rows < 2^31. */
typedef struct {
    int32_t num_tokens;  /* T: source tokens on this GPU, all simulated source ranks together */
    int32_t num_topk;    /* k: expert slots per token */
    int32_t num_experts; /* E */
    int32_t num_ranks;   /* R: simulated expert-parallel ranks */
    int32_t hidden;      /* H: channels per token */
    int32_t reserved;    /* must be 0 */
    int64_t cap_rows;    /* receive rows per rank (the guide's per-rank token capacity) */
} ep_config;

/* Output of ep_get_dispatch_layout (caller-allocated device arrays). */
typedef struct {
    int32_t *cnt_se;          /* [R][E] tokens of source rank s routed to expert e */
    int32_t *cnt_sd;          /* [R][R] tokens of source rank s with >= 1 expert on rank d */
    int32_t *recv_cnt;        /* [E] rows expert e receives */
    int32_t *expert_off;      /* [E] first row of expert e inside its rank's region */
    int32_t *rank_rows;       /* [R] rows rank d receives (may exceed cap_rows: see EP_ST_CAPACITY) */
    int32_t *src_expert_off;  /* [R][E] where the rows source rank s sends to expert e start inside rank
                                 d(e)'s region: expert_off[e] + rows of e from source ranks < s (absolute
                                 rows d*cap_rows + this + [0, cnt_se[s][e])) */
    int32_t *rank_in_expert;  /* [T][k] number of earlier tokens routed to the same expert, -1 if the slot is dropped */
    uint8_t *is_token_in_rank;/* [T][R] 1 if token t has an expert on rank d */
    /* Rank-deduplicated exchange (optional: both NULL, or both set). The
     * leader slot of (t, d) is token t's first kept slot whose expert lives
     * on rank d; rank d's rows hold its tokens in source-token order.
     * With these set, EP_ST_CAPACITY reports token_rows[d] > cap_rows
     * (the rows ep_dispatch_dedup writes) instead of rank_rows. */
    int32_t *rank_in_rank;    /* [T][k] at a leader slot: earlier tokens with a kept slot on the same rank; else -1 */
    int32_t *token_rows;      /* [R] tokens with a kept slot on rank d (its deduplicated rows) */
} ep_layout;

/* The routing state dispatch produces and combine / the backward pair reuse
 * (caller-allocated device arrays; the integer fields are set by ep_dispatch). */
typedef struct {
    int32_t *pos;     /* [T][k] receive row of slot (t, j), or -1 if the slot is dropped */
    int32_t *src_idx; /* [R*cap_rows] source token of each kept row; entries of unused rows are not written */
    int32_t num_tokens, num_topk; /* the config the handle was made for (checked by its users) */
} ep_handle;

/* Byte sizes of every caller buffer for a config (host-only, no GPU needed). */
typedef struct {
    size_t cnt_se, cnt_sd, recv_cnt, expert_off, rank_rows, src_expert_off;
    size_t rank_in_expert, is_token_in_rank, pos, src_idx;
    size_t x, recv_x_bf16, recv_x_fp8, recv_scales, recv_w, combined_x;
    size_t rank_in_rank, token_rows, recv_topk_idx, recv_topk_w; /* rank-deduplicated exchange */
    size_t workspace; /* device bytes ep_create allocates */
} ep_sizes;

/* Version of this ABI (EP_ABI_VERSION). */
int ep_version(void);

/* Text for a return code (EP_OK / EP_ERR_*). Never NULL, static storage. */
const char *ep_strerror(int code);

/* Validate a config and report buffer sizes. Host only; does not touch the
 * GPU. Returns EP_OK or EP_ERR_ARG (out may be NULL to validate only). */
int ep_query_sizes(const ep_config *cfg, ep_sizes *out);

/* Create a context on the current HIP device: validates cfg, allocates and
 * zeroes the layout workspace (the only allocation the library makes; the
 * guide's buffer is likewise created once and reused). *out is set on
 * success. Returns EP_OK, EP_ERR_ARG, EP_ERR_NOMEM or EP_ERR_HIP. */
int ep_create(const ep_config *cfg, ep_ctx **out);

/* Free the workspace (synchronizes the device first, so it must not be
 * called while a HIP graph capture is in progress). NULL is ignored. */
int ep_destroy(ep_ctx *ctx);

/* Dispatch layout from top-k routing (the step before the guide's dispatch;
 * the pages do not describe it, so its outputs are defined here):
 * per-expert and per-rank counts, the is-token-in-rank mask, and the stable
 * per-expert scan: rank_in_expert[t][j] = number of tokens t' < t routed to
 * the same expert, so every expert's rows are ordered by source token.
 * Slot validation: -1 = empty; an index outside [-1, E) sets
 * EP_ST_BAD_EXPERT and is dropped; a repeat of an expert already in the
 * token sets EP_ST_DUP_EXPERT and is dropped. rank_rows[d] > cap_rows sets
 * EP_ST_CAPACITY. One kernel launch; uses the ctx workspace.
 * topk_idx: [T][k] int32. All layout pointers must be non-NULL (T = 0 allowed)
 * except rank_in_rank and token_rows, which are computed only when both are
 * set (the rank-deduplicated exchange); rank_in_expert, is_token_in_rank and
 * rank_in_rank 16-byte aligned, the others 4-byte. */
int ep_get_dispatch_layout(ep_ctx *ctx, const int32_t *topk_idx, const ep_layout *layout,
                           ep_stream_t stream);

/* Dispatch (the guide's dispatch): for every kept slot (t, j) with expert e
 * on rank d, writes handle->pos[t][j] = d*cap_rows + expert_off[e] +
 * rank_in_expert[t][j] (slots whose row would fall at or past cap_rows are
 * dropped: pos = -1), src_idx[pos] = t, recv_w[pos] = topk_weights[t][j] and
 * the token's row:
 *   use_fp8 = 0: recv_x [R*cap_rows][H] bf16, a bit copy of x[t];
 *   use_fp8 = 1: recv_x [R*cap_rows][H] e4m3 bytes and
 *     recv_scales [R*cap_rows][H/128] fp32: per group of 128 channels,
 *     amax = max |x|, a = max(amax, 1e-4), scale = a/448, and
 *     q = e4m3(x * (448/a)) rounded to nearest even, saturating at 448
 *     (fp32 divisions and multiply, IEEE).
 * x: [T][H] bf16; topk_idx, layout: as passed to ep_get_dispatch_layout;
 * topk_weights: [T][k] fp32 (NULL: recv_w is not written; recv_w may be NULL).
 * recv_x must be 16-byte aligned; recv_scales must be non-NULL iff use_fp8.
 * Rows no slot maps to are not written. */
int ep_dispatch(ep_ctx *ctx, const uint16_t *x, const int32_t *topk_idx,
                const float *topk_weights, const ep_layout *layout, int use_fp8,
                void *recv_x, float *recv_scales, float *recv_w, ep_handle *handle,
                ep_stream_t stream);

/* ep_get_dispatch_layout followed by ep_dispatch, in one launch: the same
 * outputs (layout, handle, received rows, scales and weights), bit for bit.
 * Up to 256 tokens every dispatch block computes the whole layout in its own
 * LDS (no block waits on another); up to 4096 tokens the layout blocks raise
 * flags in the workspace and the dispatch waves, which have already loaded
 * their rows of x, wait on them only to place the rows; beyond 4096 tokens
 * the call makes the two launches it replaces (faster there). Same
 * arguments and requirements as the two calls it replaces (a layout with
 * rank_in_rank or token_rows set: EP_ERR_ARG); calls on one context are
 * ordered by the stream (two streams sharing a context race). */
int ep_dispatch_with_layout(ep_ctx *ctx, const uint16_t *x, const int32_t *topk_idx,
                            const float *topk_weights, const ep_layout *layout, int use_fp8,
                            void *recv_x, float *recv_scales, float *recv_w, ep_handle *handle,
                            ep_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as ep_dispatch_with_layout, with the same outputs bit for bit, but
 * without a context. *cfg describes the call (as for ep_create); the
 * workspace is a static device array of 4 MiB that the library holds on
 * each GPU it runs on until the process ends. The call allocates nothing
 * (no hipMalloc, no hipFree). A cfg with more than 4096 layout tiles of 256
 * tokens, or whose look-back states (tiles x (E + R) x 8 bytes) exceed the
 * 3.4 MiB the array keeps for them, returns EP_ERR_SCRATCH without
 * launching: up to about 400K tokens at 256 experts on 32 ranks, 105K at
 * 1024 experts on 64 ranks. status: a device uint32 the kernels OR their EP_ST_* bits into
 * (the caller clears it; NULL: not reported). Every call on one GPU shares
 * that GPU's array and picks up where the last call left it (the array
 * needs no clearing); calls that overlap on one GPU (two streams, two
 * threads) race and give undefined results. Same argument, alignment and
 * error rules as ep_dispatch_with_layout otherwise. */
int ep_dispatch_with_layout_noalloc(const ep_config *cfg, const uint16_t *x, const int32_t *topk_idx,
                                    const float *topk_weights, const ep_layout *layout, int use_fp8,
                                    void *recv_x, float *recv_scales, float *recv_w, ep_handle *handle,
                                    uint32_t *status, ep_stream_t stream);

/* Rank-deduplicated dispatch (the pages' normal kernels send a token once
 * per destination rank): for every leader slot (t, j) of rank d (see
 * ep_layout), writes handle->pos[t][j] = d*cap_rows + rank_in_rank[t][j]
 * (-1 if that reaches cap_rows; -1 for every slot that is not a leader),
 * src_idx[pos] = t, token t's row once (bf16 copy, or e4m3 + scales as in
 * ep_dispatch), and the row's routing entries: for every slot j' of t,
 *   recv_topk_idx[pos][j'] = e' - d*E/R and recv_topk_w[pos][j'] = topk_weights[t][j']
 * if slot j' is kept and its expert e' lives on rank d, else -1 and 0.
 * The layout must come from ep_get_dispatch_layout with rank_in_rank and
 * token_rows set. recv_topk_idx: [R*cap_rows][k] int32 (required);
 * recv_topk_w: [R*cap_rows][k] fp32 (NULL: not written; requires
 * topk_weights). The expert side then reduces each row over its local
 * experts with these weights; ep_combine with weights NULL on this handle
 * sums a token's pre-reduced rows (one per destination rank) in slot order.
 * Same stream, alignment and error rules as ep_dispatch. */
int ep_dispatch_dedup(ep_ctx *ctx, const uint16_t *x, const int32_t *topk_idx,
                      const float *topk_weights, const ep_layout *layout, int use_fp8,
                      void *recv_x, float *recv_scales, int32_t *recv_topk_idx, float *recv_topk_w,
                      ep_handle *handle, ep_stream_t stream);

/* ep_get_dispatch_layout (with rank_in_rank and token_rows, which are
 * required here) followed by ep_dispatch_dedup, in one launch: the same
 * outputs bit for bit. The layout blocks raise a flag once a tile's leader
 * rows are written and the dispatch waves, which have already loaded their
 * rows of x, wait on it only to place them (no wait for the expert totals:
 * deduplicated rows do not use them). Beyond 4096 tokens, two launches.
 * Same arguments and requirements as the two calls it replaces; calls on
 * one context are ordered by the stream. */
int ep_dispatch_dedup_with_layout(ep_ctx *ctx, const uint16_t *x, const int32_t *topk_idx,
                                  const float *topk_weights, const ep_layout *layout, int use_fp8,
                                  void *recv_x, float *recv_scales, int32_t *recv_topk_idx,
                                  float *recv_topk_w, ep_handle *handle, ep_stream_t stream);

/* Low-latency dispatch (the low-latency kernels of the DeepEP notes, section
 * 1: decode batches, a receive buffer fixed in advance, no count exchange;
 * section 5: at most 256 tokens per rank). One launch, no layout call, no
 * workspace and no block waiting on another, so it can be captured in a HIP
 * graph as it is. Receive layout: expert e owns R regions of T/R rows, region
 * s for source rank s, so rank d's rows [d*cap_rows, (d+1)*cap_rows) hold its
 * experts' regions in ascending expert order. A kept slot (t, j) of source
 * s = t / (T/R) with expert e goes to row
 *   pos[t][j] = e*T + s*(T/R) + (earlier tokens of source s routed to e)
 * (-1 for an empty, bad or repeated slot: status bits as for the layout),
 * src_idx[pos] = t; the row, scales and recv_w as in ep_dispatch.
 * recv_count: [E][R] int32, rows used in region (e, s) (required).
 * Requires cap_rows * R == E * T (every expert holds T rows) and T/R <= 256;
 * else EP_ERR_ARG. The handle works with ep_combine, ep_combine_backward and
 * ep_dispatch_backward. Rows past a region's count are not written. */
int ep_dispatch_low_latency(ep_ctx *ctx, const uint16_t *x, const int32_t *topk_idx,
                            const float *topk_weights, int use_fp8, void *recv_x, float *recv_scales,
                            float *recv_w, int32_t *recv_count, ep_handle *handle, ep_stream_t stream);

/* Combine (the guide's combine): weighted gather-reduce back to source-token
 * order. For each token t and channel i: acc = +0.0f; for j = 0..k-1 with
 * pos[t][j] >= 0: acc = fmaf(w[t][j], expert_out[pos[t][j]][i], acc) (w = 1
 * when weights is NULL); combined_x[t][i] = bf16(acc), round to nearest even.
 * expert_out: [R*cap_rows][H] bf16; weights: [T][k] fp32 or NULL;
 * combined_x: [T][H] bf16. Pointers 16-byte aligned.
 * A launch of at least 64 waves per CU (one wave per token and 1024
 * channels), on a context with no CU budget below the device's, holds each
 * of its workgroups to 40 KB of LDS it does not use, so that at most 8 of its
 * waves share a CU: kernels running beside it on the same CUs find that much
 * less LDS free. (The same holds for ep_dispatch_backward.) */
int ep_combine(ep_ctx *ctx, const uint16_t *expert_out, const ep_handle *handle,
               const float *weights, uint16_t *combined_x, ep_stream_t stream);

/* ep_combine with the fp32 sums written before rounding ([T][H] fp32), for
 * checking the reduction itself. */
int ep_combine_f32(ep_ctx *ctx, const uint16_t *expert_out, const ep_handle *handle,
                   const float *weights, float *combined_f32, ep_stream_t stream);

/* Expert-side pre-reduction of rank-deduplicated rows (the pages' normal
 * kernels send a token once per destination rank; the guide's combine brings
 * the experts' outputs back to the token's rank, [Guide] section 5). Rank d
 * sums, for each row it received, the outputs of its experts that the token
 * chose, weighted by the row's routing weights, so that ep_combine (weights
 * NULL, on the deduplicated handle) sends one row back per (token, rank).
 * expert_out: [R*cap_rows][k][H] bf16, entry (p, j) the output of received
 * row p's slot-j expert; only slots with recv_topk_idx[p][j] >= 0 are read
 * (the others may hold anything). recv_topk_idx / recv_topk_w: [R*cap_rows][k]
 * from ep_dispatch_dedup (recv_topk_w NULL: weights 1). token_rows: [R] from
 * the deduplicated layout; row p of rank d = p / cap_rows is used when
 * p - d*cap_rows < token_rows[d]. For each used row and channel i:
 *   sum = +0.0f; for j = 0 .. k-1 with recv_topk_idx[p][j] >= 0:
 *       sum = fmaf(recv_topk_w[p][j], expert_out[p][j][i], sum)
 *   reduced[p][i] = bf16_rne(sum)
 * (ep_combine's arithmetic). Unused rows of reduced are not written.
 * reduced: [R*cap_rows][H] bf16. Requires R*cap_rows*k < 2^31; rows arrays
 * 16-byte aligned. Returns EP_OK, EP_ERR_ARG, EP_ERR_ALIGN or EP_ERR_HIP.
 * ep_prereduce_f32 writes the fp32 sums instead (for checking). */
int ep_prereduce(ep_ctx *ctx, const uint16_t *expert_out, const int32_t *recv_topk_idx,
                 const float *recv_topk_w, const int32_t *token_rows, uint16_t *reduced, ep_stream_t stream);
int ep_prereduce_f32(ep_ctx *ctx, const uint16_t *expert_out, const int32_t *recv_topk_idx,
                     const float *recv_topk_w, const int32_t *token_rows, float *reduced_f32, ep_stream_t stream);

/* combine_backward (the guide: backward reuses the forward handle): the
 * gradient of combined_x travels the dispatch routes, i.e. a bf16 dispatch
 * of grad_combined [T][H] into grad_rows [R*cap_rows][H] reusing handle->pos
 * (no weights, no src_idx / recv_w writes; rows no slot maps to untouched). */
int ep_combine_backward(ep_ctx *ctx, const uint16_t *grad_combined, const ep_handle *handle,
                        uint16_t *grad_rows, ep_stream_t stream);

/* dispatch_backward (the guide: backward reuses the forward handle): a
 * gather-reduce of the per-row gradients grad_rows [R*cap_rows][H] into
 * grad_x [T][H], exactly ep_combine's arithmetic with `weights` (NULL = 1). */
int ep_dispatch_backward(ep_ctx *ctx, const uint16_t *grad_rows, const ep_handle *handle,
                         const float *weights, uint16_t *grad_x, ep_stream_t stream);

/* Synchronize `stream`, return the sticky status bits in *status and clear
 * them. Returns EP_OK or EP_ERR_HIP. */
int ep_get_status(ep_ctx *ctx, ep_stream_t stream, uint32_t *status);

/* The pages say nothing of failure detection; this is the library's own.
 * Every wait of one block on another (the layout's look-back, a fused
 * grid's readiness flags) polls at most `polls` times (0: the default,
 * 2^20; ep_create reads an initial value from the EP_SPIN_LIMIT environment
 * variable) and then gives up, setting EP_ST_TIMEOUT; the grid still ends,
 * and its workspace is re-armed for the next call on the context. Applies
 * to calls made after it returns. Returns EP_OK, or EP_ERR_ARG for a NULL
 * context. */
int ep_set_spin_limit(ep_ctx *ctx, uint32_t polls);

/* Compute-unit cap ([Notes] §2: the normal kernels can be held to a chosen
 * number of SMs so that the rest stay free for computation running beside
 * them). On this GPU the cap is a property of the stream: kernels launched on
 * the stream ep_stream_create_cus returns run only on the compute units its
 * mask enables, and the GEMM or other work that should overlap the exchange
 * runs on another stream (for instance the complementary one, exclude = 1).
 *
 * ep_cu_mask (host only, no GPU needed) fills mask[0..words) (bit i = compute
 * unit i of cu_count, 32 per word) with num_cus enabled units, num_cus/8 on
 * each of the 8 XCDs whether the hardware assigns mask bit i to XCD i mod 8
 * or to XCD i / (cu_count/8): XCD a enables units a*per + ((a*m + j) mod per),
 * j < m, with per = cu_count/8 and m = num_cus/8. exclude = 1 inverts the
 * mask (the other cu_count - num_cus units). Requires cu_count % 64 == 0,
 * 0 < num_cus <= cu_count, num_cus % 8 == 0, words >= cu_count/32, and not
 * (exclude and num_cus == cu_count); else EP_ERR_ARG.
 *
 * ep_stream_create_cus creates a default-priority HIP stream on the current
 * device with that mask (exclude = 0 and num_cus = all units: a plain
 * stream); the caller owns it and releases it with ep_stream_destroy. Any
 * ep_* call takes it as its stream; results are bit-identical on every
 * stream. */
int ep_cu_mask(int cu_count, int num_cus, int exclude, uint32_t *mask, int words);
/* The streams are blocking streams (they order with the null stream as
 * hipStreamCreate's do). ep_set_cu_budget tells a context how many compute
 * units the stream its calls run on may use (0 = all): the fused call sizes
 * the work its layout blocks take over from it, so that a capped stream does
 * not leave dispatch blocks queued behind blocks that wait. Results do not
 * depend on it. */
int ep_set_cu_budget(ep_ctx *ctx, int num_cus);
int ep_stream_create_cus(int num_cus, int exclude, ep_stream_t *out);
int ep_stream_destroy(ep_stream_t stream);

/* Measurement utility: launch `blocks` one-wave workgroups on `stream`; entry
 * b of ids (device, [blocks] uint32) receives the compute unit workgroup b
 * ran on, as (XCD id << 16) | (shader engine, array and unit bits of the
 * wave's hardware id); each workgroup then sleeps about `naps` x 3.4 us so
 * that the launch spreads over every unit the stream may use. */
int ep_cu_census(int blocks, int naps, uint32_t *ids, ep_stream_t stream);

/* Measurement utility: copy `bytes` (a multiple of 16, both pointers 16-byte
 * aligned) with a plain streaming-copy kernel, used to calibrate memory
 * counters and as the attainable-bandwidth reference. */
int ep_copy_bytes(const void *src, void *dst, size_t bytes, ep_stream_t stream);

/* Measurement utilities: the memory-access patterns of the exchange with none
 * of its arithmetic, layout or bookkeeping, timed beside the kernels as the
 * rate the HBM sustains for each pattern. They write only the buffers given;
 * the values they write are meaningless.
 *  - ep_pattern_fill: compact writes of `bytes` (a multiple of 1024) to dst,
 *    wave w storing bytes [1024w, 1024w + 1024).
 *  - ep_pattern_read: compact reads of `bytes` (a multiple of 4096) of src,
 *    4 KB per wave; sink (device, 1 uint32) is never written in practice.
 *  - ep_pattern_push: the dispatch's pattern. One wave per token loads
 *    x[t] (num_tokens x hidden bf16; hidden a multiple of 1024, at most 8192)
 *    and stores `hidden` bytes (the high byte of each channel) to row
 *    pos[t][j] of rows (num_rows x hidden bytes) for every slot with
 *    0 <= pos[t][j] < num_rows (pos: num_tokens x num_topk int32, num_topk
 *    at most 64).
 *  - ep_pattern_gather: the combine's pattern. One wave per (token,
 *    1024-channel pass) loads that pass of rows pos[t][j] of rows (num_rows
 *    x hidden bf16; slots with 0 <= pos < num_rows; num_topk at most 8) and
 *    stores their XOR to out[t] (num_tokens x hidden bf16); capped != 0
 *    launches it at the combine's residency cap (8 waves per CU).
 * Pointers to rows and vectors must be 16-byte aligned (EP_ERR_ALIGN);
 * other sizes outside these bounds return EP_ERR_ARG. */
int ep_pattern_fill(void *dst, size_t bytes, ep_stream_t stream);
int ep_pattern_read(const void *src, size_t bytes, uint32_t *sink, ep_stream_t stream);
int ep_pattern_push(const uint16_t *x, const int32_t *pos, void *rows, int num_tokens, int num_topk, int hidden,
                    int64_t num_rows, ep_stream_t stream);
int ep_pattern_gather(const uint16_t *rows, const int32_t *pos, uint16_t *out, int num_tokens, int num_topk,
                      int hidden, int64_t num_rows, int capped, ep_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */
