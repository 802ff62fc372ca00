/*
 * kda.h -- C ABI of libkda, the MI355X (gfx950) library for the Kimi Delta
 * Attention (KDA) layer path.
 *
 * The method (pages: "Kimi K3 on vLLM: Up to 370 Tokens/sec", section "Kimi
 * Delta Attention: a hybrid recurrent + full-attention stack"; "Kimi K3 +
 * vLLM: Inside the Day-0 Production Integration", section "Kimi Delta
 * Attention: When Prefix Caching Meets Recurrent State"): each KDA head keeps
 * a fixed-size d_k x d_v matrix state S and a short causal-convolution state.
 * The pages print no equation; this library computes the gated delta rule
 * with per-key-channel decay,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = scale * S_t^T q_t,
 *
 * decay first, correction against the decayed state, output from the
 * updated state.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer inside an args struct is a DEVICE pointer unless its
 *   comment says "host".  The caller owns every buffer; the library keeps no
 *   handle, allocates nothing and never synchronises the stream (except
 *   under the debug environment variable KDA_CHECK=1, which copies index
 *   arrays to the host to validate them).
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 * - Inputs dtype: KDA_BF16 or KDA_F32 (`in_dtype`), outputs `out_dtype`.
 *   Recurrent states are always fp32.  Arithmetic is fp32 (prefill products
 *   on bf16 matrix cores with split operands, fp32 accumulation).
 * - Per-token tensors are [tokens, H, d] with [H, d] contiguous; `*_stride`
 *   is the distance in ELEMENTS between consecutive tokens (0 = packed,
 *   i.e. H*d, or H for beta).  Base pointers and token strides of q, k, v,
 *   g, o must be 16-byte aligned.
 * - State pool: float [n_slots, H, d_k, d_v], d_v contiguous (row r = key
 *   channel r).  A slot index of -1 means "zero initial state" for a source
 *   and "do not write" for a destination.  Indices outside [-1, n_slots) are
 *   treated like -1 (never dereferenced).
 * - Supported sizes: d_k == d_v in {16, 32, 64, 128}; H >= 1.
 * - Status: every call returns a kda_status; KDA_OK means the work was
 *   enqueued.  kda_last_error() gives a one-line reason for the calling
 *   thread's last failure.  n_seq == 0 is a no-op returning KDA_OK.
 * - Preconditions on device data that cannot be checked without a sync
 *   (checked only under KDA_CHECK=1): cu_seqlens non-decreasing and within
 *   [0, T_tot]; no source slot of one sequence equals a destination or
 *   checkpoint slot of another sequence in the same call (two sequences that
 *   share a cached prefix must take their copies in separate calls).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 2

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* a required pointer is NULL */
    KDA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
    KDA_ERR_DTYPE = 3,       /* unknown dtype code */
    KDA_ERR_ALIGN = 4,       /* pointer/stride not 16-byte aligned, or a
                                checkpoint interval not a multiple of chunk */
    KDA_ERR_WORKSPACE = 5,   /* workspace missing or too small */
    KDA_ERR_UNSUPPORTED = 6, /* valid request outside what is built */
    KDA_ERR_HIP = 7,         /* the HIP runtime reported an error */
    KDA_ERR_ARG = 8,         /* malformed argument struct or invalid data
                                (KDA_CHECK=1 validation) */
    KDA_ERR_CAPACITY = 9     /* a host output array is too small */
} kda_status;

typedef enum kda_dtype { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype;

typedef void *kda_stream_t; /* hipStream_t */

/* Short human-readable name of a status code (static string). */
const char *kda_status_str(int status);
/* KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);
/* One-line reason for the calling thread's most recent non-OK status. */
const char *kda_last_error(void);
/* sizeof() of each args struct as compiled into the library: which = 0 conv,
 * 1 prefill, 2 decode, 3 verify, 4 decode_conv, 5 verify_conv, 6 plan,
 * 7 prefill_conv.  Returns 0 for other values. */
size_t kda_args_sizeof(int which);

/* ------------------------------------------------------------------------
 * kda_conv_short -- short causal depthwise convolution with carried state.
 *
 * The KDA layer runs a short causal convolution on its q/k/v channels and
 * carries its state across calls (Day-0 Integration page, section "Kimi
 * Delta Attention: When Prefix Caching Meets Recurrent State"; the fused
 * decode kernel folds it in, section "Separate Prefill/Decode Code Paths").
 *
 *   y[t, c] = bias[c] + sum_{j=0}^{W-1} weight[c, j] * xbar[t - (W-1) + j, c]
 *   (then SiLU when act == 1)
 *
 * where xbar is the sequence's carried state (last W-1 raw inputs, oldest
 * first; zeros when src_slot < 0) followed by its tokens.  Tap W-1 multiplies
 * the current token.  The new state (the last W-1 raw inputs after
 * advance_len[s] tokens, or after all tokens when advance_len is NULL) is
 * written to dst_slot[s] when >= 0; src == dst (in place) is allowed.
 * Outputs are produced for every token.  Sequences may be empty.
 *
 * Optional per-head normalisation (the q / k step of the fused order,
 * kda_prefill_varlen_conv): with norm_d > 0 every token's channels
 * [0, norm_channels) are taken in groups of norm_d and each group is divided
 * by sqrt(sum of its squares + norm_eps), after the SiLU; the channels past
 * norm_channels keep their values.  norm_d in {16, 32, 64, 128},
 * norm_channels a multiple of norm_d and <= C, W <= 4 (else
 * KDA_ERR_UNSUPPORTED / KDA_ERR_ARG); y is then rounded to dtype once.
 * ---------------------------------------------------------------------- */
typedef struct kda_conv_args {
    size_t struct_size;          /* sizeof(kda_conv_args) */
    const void *x;               /* [T_tot, C], row stride x_stride */
    void *y;                     /* [T_tot, C], row stride y_stride */
    const void *weight;          /* [C, W] contiguous */
    const void *bias;            /* [C] or NULL */
    const int32_t *cu_seqlens;   /* [n_seq + 1] token offsets into x / y */
    void *conv_pool;             /* [n_slots, C, W-1] contiguous (channel-major) */
    const int32_t *src_slot;     /* [n_seq]; -1 = zero history */
    const int32_t *dst_slot;     /* [n_seq]; -1 = do not write */
    const int32_t *advance_len;  /* [n_seq] or NULL; clamped to [0, len] */
    int64_t x_stride;            /* elements between tokens (0 = C) */
    int64_t y_stride;            /* elements between tokens (0 = C) */
    int64_t T_tot;               /* rows of x and y */
    int64_t n_slots;
    int32_t n_seq;
    int32_t C;                   /* channels; multiple of 16 / sizeof(dtype) */
    int32_t W;                   /* 2..8 */
    int32_t dtype;               /* x, y, weight, bias and conv_pool */
    int32_t act;                 /* 0 none, 1 SiLU */
    int32_t norm_d;              /* 0 = no normalisation, else the group size */
    int64_t norm_channels;       /* channels normalised (from channel 0) */
    float norm_eps;              /* >= 0 */
    int32_t reserved;
} kda_conv_args;

int kda_conv_short(const kda_conv_args *args, kda_stream_t stream);

/* ------------------------------------------------------------------------
 * kda_ckpt_plan -- where interval checkpoints fall (host-only integer work).
 *
 * Interval retention (Day-0 Integration page, section "Interval-Based and
 * Marconi-Style Retention"): a state snapshot is kept every `interval`
 * tokens.  A sequence occupying absolute positions [start, start + len) gets
 * one checkpoint for every multiple p of `interval` with start < p <
 * start + len: the state after its first p - start tokens.  The final state
 * is not a checkpoint (kda_prefill_varlen returns it through dst_slot).
 * Count per sequence: floor((start + len - 1) / interval) - floor(start /
 * interval) (0 when len == 0).
 *
 *   cu_seqlens   host [n_seq + 1]
 *   start_pos    host [n_seq] absolute start of each sequence, or NULL (0)
 *   interval     > 0 and a multiple of `chunk` (else KDA_ERR_ALIGN)
 *   chunk        16, 32 or 64 (the prefill chunk the plan is for)
 *   ckpt_cu      host [n_seq + 1] out: prefix counts
 *   ckpt_pos     host [cap] out: positions, sequence by sequence (may be
 *                NULL when cap == 0, to query the total)
 *   n_total      host out: total number of checkpoints
 * Returns KDA_ERR_CAPACITY (after filling ckpt_cu and n_total) when the
 * total exceeds cap.
 * ---------------------------------------------------------------------- */
int kda_ckpt_plan(const int32_t *cu_seqlens, const int32_t *start_pos, int32_t n_seq,
                  int32_t interval, int32_t chunk, int32_t *ckpt_cu, int32_t *ckpt_pos,
                  int32_t cap, int32_t *n_total);

/* ------------------------------------------------------------------------
 * kda_ckpt_plan_device -- the checkpoint plan of kda_ckpt_plan, built on the
 * device from device cu_seqlens, with checkpoint slots taken from a device
 * free list.
 *
 * The Day-0 Integration page (section "Separate Prefill/Decode Code Paths")
 * reports per-batch metadata preparation as a batch-1 bottleneck and moves
 * it into dedicated kernels.  This call keeps the checkpoint table of
 * interval retention (same page, section "Agentic Serving: Cache Retention
 * Across Turns") off the host: two small kernels whose launch shapes depend
 * only on n_seq and cap, no allocation and no synchronisation, so it can be
 * recorded in a HIP graph together with kda_prefill_varlen.
 *
 * Per sequence s, with the clamping kda_prefill_varlen applies
 * (bos = clamp(cu[s], 0, T_tot), eos = clamp(cu[s+1], bos, T_tot),
 * len = eos - bos, start = max(start_pos[s], 0)):
 *   count(s)     = len > 0 ? floor((start+len-1)/interval) - floor(start/interval) : 0
 *   ckpt_cu      exclusive prefix sums of count, ckpt_cu[0] = 0
 *   ckpt_pos[i]  = (floor(start/interval) + 1 + i - ckpt_cu[s]) * interval
 *                  for ckpt_cu[s] <= i < ckpt_cu[s+1]
 *   ckpt_slot[i] = free_slots[i] for i < n_free, else -1 (a slot of -1 makes
 *                  kda_prefill_varlen skip that checkpoint)
 *   n_total[0]   = ckpt_cu[n_seq]
 * Entries i >= cap of ckpt_pos / ckpt_slot are not written; pass the same
 * cap as kda_prefill_args.n_ckpt and the prefill skips checkpoints past it.
 * Counts saturate at 2^31 - 1.  n_seq == 0 still writes ckpt_cu[0] = 0
 * and n_total.  For valid inputs (lengths >= 0, starts
 * >= 0) the table equals the one kda_ckpt_plan builds on the host.
 * ---------------------------------------------------------------------- */
typedef struct kda_plan_args {
    size_t struct_size;          /* sizeof(kda_plan_args) */
    const int32_t *cu_seqlens;   /* [n_seq + 1] */
    const int32_t *start_pos;    /* [n_seq] absolute start, or NULL (all 0) */
    const int32_t *free_slots;   /* [n_free] pool slots, or NULL when n_free == 0 */
    int32_t *ckpt_cu;            /* [n_seq + 1] out */
    int32_t *ckpt_pos;           /* [cap] out, or NULL */
    int32_t *ckpt_slot;          /* [cap] out, or NULL */
    int32_t *n_total;            /* [1] out, or NULL: total checkpoints (may exceed cap) */
    int64_t T_tot;               /* tokens of the packed batch (>= 0) */
    int32_t n_seq;               /* >= 0 */
    int32_t interval;            /* > 0 and a multiple of chunk (else KDA_ERR_ALIGN) */
    int32_t chunk;               /* 16, 32 or 64 */
    int32_t cap;                 /* >= 0: capacity of ckpt_pos / ckpt_slot */
    int32_t n_free;              /* >= 0: length of free_slots */
    int32_t reserved;
} kda_plan_args;

int kda_ckpt_plan_device(const kda_plan_args *args, kda_stream_t stream);

/* ------------------------------------------------------------------------
 * kda_prefill_varlen -- chunked prefill of packed sequences.
 *
 * Runs the recurrence over each sequence of a packed batch (cu_seqlens),
 * starting from src_slot's state (or zero), writing every token's output,
 * the final state to dst_slot, and interval checkpoints to ckpt_slot (the
 * positions of kda_ckpt_plan, echoed in ckpt_pos_out).  This is how a
 * long shared prompt's state snapshots are registered for prefix reuse and
 * copied into a private destination before extension (Day-0 Integration
 * page, section "Separating Physical Blocks, Scheduler Alignment, and
 * Prefix Matching"): src is only read, never written.
 *
 * Chunk boundaries are aligned to absolute positions (multiples of chunk),
 * so a sequence may start mid-chunk; checkpoints therefore always fall on
 * chunk boundaries.
 *
 * Segment scan.  A sequence longer than segment_len tokens is split at
 * the absolute multiples of segment_len into segments that run in parallel:
 * every segment runs with outputs and checkpoints from a zero state (the
 * first segment: from its true initial state, which makes it final), ending
 * in its state S_loc; every later segment also computes its transition M
 * (the same recurrence applied to S = I with v = 0), which stops once M is
 * exactly zero (it stays zero from there on).  Then
 * S_in(j+1) = M_j S_in(j) + S_loc(j) chains the segments (fp32), and every
 * later segment reruns from its S_in the chunks before its M became zero
 * (all of them if it never did), overwriting those outputs and checkpoints;
 * past that point the zero-started state is the state.  The result is the
 * same function of the inputs as the unsplit run (up to rounding).  The
 * split needs the workspace: its size comes from kda_prefill_workspace_bytes
 * for the same args (0 when T_tot <= segment_len, since nothing can be
 * split then).  segment_len: 0 = the library default (32768), < 0 = never
 * split, > 0 = that length, a multiple of chunk (else KDA_ERR_ALIGN).
 *
 * In place: src_slot[s] == dst_slot[s] is allowed, also for split
 * sequences (the final state is written only after every segment has read
 * its starting state).
 *
 * With T_tot == 0 the per-token pointers (q, k, v, g, beta, o) may be NULL:
 * every sequence is empty, and only the final states (the source states)
 * are written.
 *
 * Decay range (precondition).  The chunked form scales the rows of a tile
 * (32 tokens at absolute multiples of 32; 16 when chunk == 16) by
 * exp(+-(G_r - G_15)), G being the running sum of g over the tile's rows.
 * Results are exact to the stated tolerance while every such exponent stays
 * within +-80 (nats) for every key channel -- e.g. whenever each g lies in
 * [-5, 0], or isolated tokens reach far lower (a single -20 is fine).
 * Beyond it a factor leaves the fp32 range and outputs and states may be
 * non-finite.  Checked under KDA_CHECK=1 (KDA_ERR_ARG naming the sequence,
 * head, channel and tile).
 * ---------------------------------------------------------------------- */
typedef struct kda_prefill_args {
    size_t struct_size;          /* sizeof(kda_prefill_args) */
    const void *q;               /* [T_tot, H, d_k] */
    const void *k;               /* [T_tot, H, d_k] */
    const void *v;               /* [T_tot, H, d_v] */
    const void *g;               /* [T_tot, H, d_k] log decay (alpha = exp g) */
    const void *beta;            /* [T_tot, H] */
    void *o;                     /* [T_tot, H, d_v] out_dtype */
    const int32_t *cu_seqlens;   /* [n_seq + 1] */
    float *state_pool;           /* [n_slots, H, d_k, d_v] */
    const int32_t *src_slot;     /* [n_seq]; -1 = zero initial state */
    const int32_t *dst_slot;     /* [n_seq]; -1 = final state not written */
    const int32_t *start_pos;    /* [n_seq] absolute start, or NULL (all 0) */
    const int32_t *ckpt_cu;      /* [n_seq + 1] from kda_ckpt_plan, or NULL */
    const int32_t *ckpt_slot;    /* [n_ckpt] pool slot of each checkpoint */
    int32_t *ckpt_pos_out;       /* [n_ckpt] or NULL: position written */
    void *workspace;             /* scratch of workspace_bytes, or NULL */
    int64_t q_stride, k_stride, v_stride, g_stride, beta_stride, o_stride; /* 0 = packed */
    int64_t T_tot;
    int64_t n_slots;
    int64_t workspace_bytes;
    int64_t n_ckpt;              /* length of ckpt_slot / ckpt_pos_out */
    int32_t n_seq;
    int32_t H, d_k, d_v;
    int32_t chunk;               /* 16, 32 or 64 */
    int32_t in_dtype, out_dtype;
    int32_t ckpt_interval;       /* 0 = no checkpoints; multiple of chunk */
    float scale;
    int32_t segment_len;         /* segment scan length: 0 default, < 0 off */
} kda_prefill_args;

/* Workspace bytes kda_prefill_varlen needs for these args (host-only). */
int64_t kda_prefill_workspace_bytes(const kda_prefill_args *args);
int kda_prefill_varlen(const kda_prefill_args *args, kda_stream_t stream);

/* ------------------------------------------------------------------------
 * kda_prefill_varlen_conv -- the prefill from the tokens' raw projections.
 *
 * The prefill side of the layer's fused order (Day-0 Integration page,
 * section "Separate Prefill/Decode Code Paths": the short causal conv over
 * the q / k / v projections in front of the recurrence; section "Kimi Delta
 * Attention: When Prefix Caching Meets Recurrent State" for the conv state
 * a prefix snapshot carries).  Per sequence s of the packed batch:
 *   y = conv(history ++ tokens) (+ SiLU when act == 1), channel c:
 *       y[t, c] = bias[c] + sum_{j<W} w[c, j] xbar[t - (W-1) + j, c]
 *   q, k, v = the three channel blocks of y, each [H, d]
 *   qk_l2norm: q <- q / sqrt(|q|^2 + norm_eps) per token and head, k alike
 *   q, k, v rounded once to in_dtype and written to `qkv`
 *   then kda_varlen of `prefill` on those q, k, v.
 * The conv history of s is read from conv_pool[conv_src_slot[s]] (zeros when
 * -1) and the last W-1 raw inputs of history ++ tokens are written to
 * conv_pool[conv_dst_slot[s]] (not when -1); src == dst is allowed.
 * With conv_ckpt_slot, every interval checkpoint j of the prefill (the
 * positions and table of kda_ckpt_plan) also gets the conv history a run
 * resumed there needs -- the W-1 raw inputs of history ++ tokens before the
 * checkpoint's position -- in conv_pool[conv_ckpt_slot[j]] (not when -1 or
 * out of range): with the recurrent checkpoint it makes the snapshot a
 * prefix hit resumes from.  Checkpoint conv slots must differ from every
 * conv source and destination slot of the call.
 *
 * Two launches on `stream`: the conv with the normalisation (one streaming
 * pass over x that writes qkv), then the chunked prefill reading qkv.  The
 * prefill kernel holds its whole register file and LDS for the chunk
 * pipeline, so the conv is not folded into its tile loads.
 *
 * Layout: x [T_tot, 3 H d] in_dtype (row stride x_stride; 0 = 3 H d),
 * conv_weight [3 H d, W], conv_bias [3 H d] or NULL, conv_pool
 * [n_conv_slots, 3 H d, W-1] in_dtype; qkv [T_tot, 3 H d] in_dtype packed,
 * caller-owned (also an output: the q | k | v the recurrence consumed).
 * `prefill` is a kda_prefill_args with q, k and v NULL and their strides 0
 * (the library points them into qkv), d_k == d_v == d; every other field
 * as kda_prefill_varlen (g, beta, o, slots, checkpoints, workspace from
 * kda_prefill_workspace_bytes of the same args, segment_len).
 * With T_tot == 0, x and qkv may be NULL (and the per-token pointers of
 * `prefill`, as in kda_prefill_varlen): nothing is read from them; the conv
 * histories and the final states are still copied to their destinations.
 * Errors: those of kda_prefill_varlen, raised before anything is launched;
 * q / k / v given or d_k != d_v -> KDA_ERR_ARG; conv_ckpt_slot without
 * checkpoints (ckpt_interval 0) -> KDA_ERR_ARG; W outside 2..4 ->
 * KDA_ERR_UNSUPPORTED; qkv smaller than T_tot * 3 H d elements ->
 * KDA_ERR_WORKSPACE; x, qkv, conv_weight or conv_pool not 16-byte aligned,
 * or an x stride that breaks 16-byte rows -> KDA_ERR_ALIGN; act not 0/1,
 * qk_l2norm not 0/1 or norm_eps < 0 -> KDA_ERR_ARG.
 * ---------------------------------------------------------------------- */
typedef struct kda_prefill_conv_args {
    size_t struct_size;          /* sizeof(kda_prefill_conv_args) */
    kda_prefill_args prefill;    /* q, k, v NULL; see above */
    const void *x;               /* [T_tot, 3 H d] raw q | k | v projections */
    const void *conv_weight;     /* [3 H d, W] */
    const void *conv_bias;       /* [3 H d] or NULL */
    void *conv_pool;             /* [n_conv_slots, 3 H d, W-1] in_dtype */
    const int32_t *conv_src_slot;/* [n_seq]; -1 = zero history */
    const int32_t *conv_dst_slot;/* [n_seq]; -1 = not written */
    const int32_t *conv_ckpt_slot; /* [n_ckpt] conv slot of each checkpoint, or NULL */
    void *qkv;                   /* [T_tot, 3 H d] in_dtype, packed */
    int64_t x_stride;            /* elements between tokens of x (0 = 3 H d) */
    int64_t n_conv_slots;
    int64_t qkv_bytes;           /* size of qkv in bytes */
    int32_t W;                   /* 2..4 */
    int32_t act;                 /* 0 none, 1 SiLU */
    int32_t qk_l2norm;           /* 0 / 1 */
    float norm_eps;              /* >= 0 */
} kda_prefill_conv_args;

int kda_prefill_varlen_conv(const kda_prefill_conv_args *args, kda_stream_t stream);

/* ------------------------------------------------------------------------
 * kda_prefill_varlen_noalloc -- kda_prefill_varlen for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, results and errors as kda_prefill_varlen, except:
 * - `workspace` must be NULL and `workspace_bytes` 0 (else KDA_ERR_ARG):
 *   the segment scan uses a scratch array of kda_prefill_noalloc_max_bytes()
 *   bytes (64 MiB) that the library holds on every GPU it runs on until the
 *   process ends.  A call whose split needs more (kda_prefill_workspace_bytes
 *   of the same args) returns KDA_ERR_WORKSPACE and launches nothing; calls
 *   that split nothing (T_tot <= segment_len, or segment_len < 0) need none.
 *   At H = 16, d = 128 the limit admits T_tot up to about 6.6 segment
 *   lengths.
 * - Nothing in the scratch has to start at zero; every call on a GPU shares
 *   that GPU's array and leaves its own contents in it, so calls that
 *   overlap on one GPU (different streams, or host threads) race and must
 *   be ordered by the caller.
 * - The stream must belong to the current device (the scratch address is
 *   the current device's).
 * - No KDA_CHECK=1 validation (it would allocate host buffers).
 * ---------------------------------------------------------------------- */
int kda_prefill_varlen_noalloc(const kda_prefill_args *args, kda_stream_t stream);
/* Bytes of the scratch array kda_prefill_varlen_noalloc uses (host-only). */
int64_t kda_prefill_noalloc_max_bytes(void);

/* ------------------------------------------------------------------------
 * kda_decode -- one token per sequence, state updated in place.
 *
 * The decode step of the KDA layer (Day-0 Integration page, section
 * "Separate Prefill/Decode Code Paths"; "Kimi K3 on vLLM", section "Kimi
 * Delta Attention: a hybrid recurrent + full-attention stack", where decode
 * runs a fused kernel): for sequence s the state is read from src_slot[s],
 * advanced by one token and written to dst_slot[s] (usually the same slot).
 * ---------------------------------------------------------------------- */
typedef struct kda_decode_args {
    size_t struct_size;          /* sizeof(kda_decode_args) */
    const void *q, *k, *v, *g;   /* [n_seq, H, d] */
    const void *beta;            /* [n_seq, H] */
    void *o;                     /* [n_seq, H, d_v] out_dtype */
    float *state_pool;           /* [n_slots, H, d_k, d_v] */
    const int32_t *src_slot;     /* [n_seq] */
    const int32_t *dst_slot;     /* [n_seq] */
    int64_t q_stride, k_stride, v_stride, g_stride, beta_stride, o_stride; /* 0 = packed */
    int64_t n_slots;
    int32_t n_seq;
    int32_t H, d_k, d_v;
    int32_t in_dtype, out_dtype;
    float scale;
    int32_t reserved;
} kda_decode_args;

int kda_decode(const kda_decode_args *args, kda_stream_t stream);

/* ------------------------------------------------------------------------
 * kda_decode_conv -- the decode step with the short convolution fused in.
 *
 * The KDA decode kernel runs the q/k/v short convolution and the recurrence
 * in one launch ("Kimi K3 on vLLM", section "Kimi Delta Attention: a hybrid
 * recurrent + full-attention stack"; Day-0 Integration page, section
 * "Separate Prefill/Decode Code Paths").  For sequence s and head h:
 *
 *   xbar[c]  = conv state of channel c (W-1 raw inputs, oldest first) ++ x[s, c]
 *   y[c]     = bias[c] + sum_j weight[c, j] * xbar[c][j]   (+ SiLU when act = 1)
 *   q, k, v  = the head-h slices of the q, k and v blocks of y (fp32, unrounded)
 *   qk_l2norm: q <- q / sqrt(|q|^2 + norm_eps), k likewise
 *   then the kda_decode step with g[s, h], beta[s, h]:
 *   S <- Diag(exp g) S;  S <- S + beta k (v - S^T k)^T;  o = scale S^T q.
 *   With out_gate (the output gate the fused kernel folds in, section
 *   "Separate Prefill/Decode Code Paths"; the pages name it without a
 *   formula -- this library reads it as a gated RMS norm per head):
 *   o <- o / sqrt(mean_c o[c]^2 + out_norm_eps) * out_norm_weight[c]
 *        * sigmoid(out_gate[s, h, c])        (the mean over the d channels)
 *
 * Channels of x, weight, bias and the conv pool are ordered [q block | k
 * block | v block], each block [H, d] (C = 3 H d).  The conv state of the
 * sequence advances by the token (xbar[1..W-1] to conv_dst_slot; -1 = no
 * write; conv_src_slot -1 = zero history); the recurrent state goes from
 * src_slot to dst_slot as in kda_decode.  Each (sequence, head) reads and
 * writes only its own channels and state, so in-place slots are race free.
 *
 *   x            [n_seq, 3 H d] in_dtype, row stride x_stride (0 = packed)
 *   conv_weight  [3 H d, W] in_dtype;  conv_bias [3 H d] or NULL
 *   conv_pool    [n_conv_slots, 3 H d, W-1] in_dtype
 *   g [n_seq, H, d], beta [n_seq, H] in_dtype; o [n_seq, H, d] out_dtype
 *   state_pool   fp32 [n_slots, H, d, d]
 *   out_gate     [n_seq, H, d] in_dtype, row stride out_gate_stride (0 =
 *                packed), or NULL (o as computed); out_norm_weight [d]
 *                in_dtype, shared by the heads, required with out_gate
 * Errors: W outside 2..4 -> KDA_ERR_UNSUPPORTED; d not 16/32/64/128 ->
 * KDA_ERR_UNSUPPORTED; x, conv_weight, conv_bias (when given), conv_pool,
 * g, o, state_pool, out_gate or out_norm_weight not 16-byte aligned, or an
 * x or out_gate stride that breaks 16-byte rows -> KDA_ERR_ALIGN; act not
 * 0/1, qk_l2norm not 0/1, norm_eps or out_norm_eps < 0 -> KDA_ERR_ARG;
 * out_gate without out_norm_weight -> KDA_ERR_NULL.
 * ---------------------------------------------------------------------- */
typedef struct kda_decode_conv_args {
    size_t struct_size;          /* sizeof(kda_decode_conv_args) */
    const void *x;               /* [n_seq, 3 H d] raw projections of the token */
    const void *conv_weight;     /* [3 H d, W] */
    const void *conv_bias;       /* [3 H d] or NULL */
    void *conv_pool;             /* [n_conv_slots, 3 H d, W-1] */
    const int32_t *conv_src_slot; /* [n_seq]; -1 = zero history */
    const int32_t *conv_dst_slot; /* [n_seq]; -1 = do not write */
    const void *g;               /* [n_seq, H, d] */
    const void *beta;            /* [n_seq, H] */
    void *o;                     /* [n_seq, H, d] out_dtype */
    float *state_pool;           /* [n_slots, H, d, d] */
    const int32_t *src_slot;     /* [n_seq] */
    const int32_t *dst_slot;     /* [n_seq] */
    int64_t x_stride, g_stride, beta_stride, o_stride; /* per sequence; 0 = packed */
    int64_t n_slots;
    int64_t n_conv_slots;
    int32_t n_seq;
    int32_t H, d;
    int32_t W;                   /* conv width, 2..4 */
    int32_t act;                 /* 0 none, 1 SiLU */
    int32_t qk_l2norm;           /* 0 / 1 */
    float norm_eps;              /* >= 0 */
    int32_t in_dtype, out_dtype;
    float scale;
    const void *out_gate;        /* [n_seq, H, d] or NULL: no output gate / norm */
    const void *out_norm_weight; /* [d]; required with out_gate */
    int64_t out_gate_stride;     /* per sequence; 0 = packed (H d) */
    float out_norm_eps;          /* >= 0 */
    int32_t reserved;
} kda_decode_conv_args;

int kda_decode_conv(const kda_decode_conv_args *args, kda_stream_t stream);

/* ------------------------------------------------------------------------
 * kda_verify_conv -- speculative verification with the short convolution
 * fused in.
 *
 * kda_verify on q, k, v formed as in kda_decode_conv from the T_spec
 * tokens' raw projections: the conv runs over (conv history ++ the tokens),
 * q and k are normalised per token and head when qk_l2norm.  The accepted
 * length commits both states: the recurrent state after L tokens to
 * dst_slot and the conv history after L tokens (the W-1 raw inputs ending
 * at token L-1) to conv_dst_slot.  Modes, accepted_len semantics and
 * committed_len_out as kda_verify (outputs-only calls write neither state).
 *
 *   x   [n_seq, T_spec, 3 H d] in_dtype, token stride x_stride (0 = packed;
 *       sequence stride T_spec * x_stride)
 *   g   [n_seq, T_spec, H, d], beta [n_seq, T_spec, H], o [n_seq, T_spec, H, d]
 *   out_gate [n_seq, T_spec, H, d] (token stride out_gate_stride) or NULL:
 *       every output position passes through the gated RMS norm of
 *       kda_decode_conv
 *   other arguments as kda_decode_conv.
 * Errors as kda_decode_conv; T_spec outside 1..16 -> KDA_ERR_SHAPE.
 * ---------------------------------------------------------------------- */
typedef struct kda_verify_conv_args {
    size_t struct_size;          /* sizeof(kda_verify_conv_args) */
    const void *x;               /* [n_seq, T_spec, 3 H d] raw projections */
    const void *conv_weight;     /* [3 H d, W] */
    const void *conv_bias;       /* [3 H d] or NULL */
    void *conv_pool;             /* [n_conv_slots, 3 H d, W-1] */
    const int32_t *conv_src_slot; /* [n_seq]; -1 = zero history */
    const int32_t *conv_dst_slot; /* [n_seq]; -1 = do not write */
    const void *g;               /* [n_seq, T_spec, H, d] */
    const void *beta;            /* [n_seq, T_spec, H] */
    void *o;                     /* [n_seq, T_spec, H, d] out_dtype, or NULL */
    float *state_pool;           /* [n_slots, H, d, d] */
    const int32_t *src_slot;     /* [n_seq] */
    const int32_t *dst_slot;     /* [n_seq] */
    const int32_t *accepted_len; /* [n_seq] or NULL */
    int32_t *committed_len_out;  /* [n_seq] or NULL */
    int64_t x_stride, g_stride, beta_stride, o_stride; /* per token; 0 = packed */
    int64_t n_slots;
    int64_t n_conv_slots;
    int32_t n_seq;
    int32_t T_spec;              /* 1..16 */
    int32_t H, d;
    int32_t W;                   /* conv width, 2..4 */
    int32_t act;                 /* 0 none, 1 SiLU */
    int32_t qk_l2norm;           /* 0 / 1 */
    float norm_eps;              /* >= 0 */
    int32_t in_dtype, out_dtype;
    float scale;
    int32_t reserved;
    const void *out_gate;        /* [n_seq, T_spec, H, d] or NULL */
    const void *out_norm_weight; /* [d]; required with out_gate */
    int64_t out_gate_stride;     /* per token; 0 = packed (H d) */
    float out_norm_eps;          /* >= 0 */
    int32_t reserved2;
} kda_verify_conv_args;

int kda_verify_conv(const kda_verify_conv_args *args, kda_stream_t stream);

/* ------------------------------------------------------------------------
 * kda_verify -- speculative verification with a commit at the accepted
 * length.
 *
 * Speculative decoding proposes several draft tokens that the target model
 * verifies in one parallel pass ("Kimi K3 on vLLM", section "Ultra-low
 * latency: speculative decoding with DSpark"; the KDA backend runs a separate
 * path for it, section "Kimi Delta Attention: a hybrid recurrent +
 * full-attention stack").  Each sequence holds T_spec tokens (position 0 =
 * the last accepted token, then the drafts), laid out [n_seq, T_spec, H, d]
 * with token stride *_stride (sequence stride = T_spec * token stride).
 *
 * Modes:
 *   o != NULL, accepted_len == NULL : outputs for all T_spec positions; the
 *                                     pool is not written.
 *   o == NULL, accepted_len != NULL : commit only: the state after exactly
 *                                     accepted_len[s] tokens goes to
 *                                     dst_slot[s].
 *   both                            : fused (outputs + commit in one pass).
 * accepted_len[s] = L counts tokens including position 0; L = 0 commits the
 * source state unchanged; L outside [0, T_spec] rejects the sequence:
 * committed_len_out[s] = -1 and dst is not written.  Otherwise
 * committed_len_out[s] = L.  Outputs at positions >= L are still produced
 * from the running state.
 * ---------------------------------------------------------------------- */
typedef struct kda_verify_args {
    size_t struct_size;          /* sizeof(kda_verify_args) */
    const void *q, *k, *v, *g;   /* [n_seq, T_spec, H, d] */
    const void *beta;            /* [n_seq, T_spec, H] */
    void *o;                     /* [n_seq, T_spec, H, d_v] or NULL */
    float *state_pool;           /* [n_slots, H, d_k, d_v] */
    const int32_t *src_slot;     /* [n_seq] */
    const int32_t *dst_slot;     /* [n_seq] */
    const int32_t *accepted_len; /* [n_seq] or NULL */
    int32_t *committed_len_out;  /* [n_seq] or NULL */
    int64_t q_stride, k_stride, v_stride, g_stride, beta_stride, o_stride; /* per token; 0 = packed */
    int64_t n_slots;
    int32_t n_seq;
    int32_t T_spec;              /* 1..16 */
    int32_t H, d_k, d_v;
    int32_t in_dtype, out_dtype;
    float scale;
} kda_verify_args;

int kda_verify(const kda_verify_args *args, kda_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
