/*
 * finch_wkv.h -- C ABI of the Finch WKV pre-fill library (libfinch_wkv.so).
 *
 * The operation (GoldFinch architecture summary page, section 3.4 "Finch-C2
 * Time Mixing", paragraph "Recurrent state update and output", with base
 * Finch's static bonus u from modification (4) of the same section):
 *
 *   per (sequence n, head h), tokens t = 0 .. L_n - 1 in order,
 *     o_t[j]   = sum_i r_t[i] * ( S[i][j] + u[h][i] * k_t[i] * v_t[j] )
 *     S[i][j] <- w_t[i] * S[i][j] + k_t[i] * v_t[j]
 *   starting from S = state_in[n][h] (zeros when state_in is NULL) and ending
 *   with state_out[n][h] = S.  Rows i of S are key channels (the decay acts on
 *   them), columns j are value channels.  This is the recurrent pre-fill of
 *   the Finch layers: a whole submitted context is consumed at O(1) cost per
 *   token and leaves a fixed-size state that later tokens continue from
 *   (abstract; section 3.4 "Training and Inference Procedures", inference
 *   pre-fill).  Carrying state_out into the next call as state_in continues
 *   the same sequence exactly.  Calls in which no sequence has more than 16
 *   tokens -- recurrent generation steps continuing a pre-filled state --
 *   compute the same result with a kernel built to stream the states, which
 *   are then most of the traffic.
 *
 * Layouts (all row-major, D fastest, no padding):
 *   r, k, v, w : [B, T, H, D] (fixed length) or [total_tokens, H, D] (packed)
 *                element type `in_dtype` (WKV_BF16 or WKV_F32)
 *   u          : [H, D] fp32
 *   o          : same layout as r, fp32
 *   state_in   : [B or N, H, D, D] fp32, [i][j] = [key channel][value channel]
 *   state_out  : same as state_in
 * Supported head size: D = 64.
 *
 * Ownership and concurrency: the caller owns every buffer.  All tensor
 * pointers are DEVICE pointers, except cu_seqlens_host.  The library never
 * allocates device memory; scratch lives in the caller's `workspace`.  Calls
 * are asynchronous on `stream` (a hipStream_t; NULL = the null stream): when a
 * call returns WKV_OK the work is enqueued, and inputs must stay valid and
 * unmodified until it completes.  Kernel faults surface at the caller's next
 * synchronisation.  Two calls that share a workspace must be ordered (same
 * stream, or synchronised).
 *
 * Aliasing: state_out == state_in (exact same pointer) is allowed -- the
 * carried-state idiom.  Any other overlap between an output (o, state_out)
 * and any other buffer is rejected with WKV_EINVAL (checked on the address
 * ranges).
 *
 * Domain: 0 < w <= 1 (w == 1 exactly is legal); any d, including +-inf, with
 * WKV_FLAG_DECAY_LOG.  Values outside it and NaN are not checked and
 * propagate.  Finite |r|, |k| below 2^31 are required
 * (the chunked evaluation rescales them by decay factors up to 2^96).
 *
 * Errors: every entry point validates its arguments before touching the GPU
 * and returns a wkv_status_t; wkv_last_error() gives a human-readable detail
 * for the calling thread.  No exception crosses the ABI.  Nothing is written
 * when a call fails validation.
 */
#ifndef FINCH_WKV_H
#define FINCH_WKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FINCH_WKV_ABI_VERSION 5

/* Bytes of control records at the start of every nonzero workspace (see
 * wkv_prefill_workspace_bytes). */
#define WKV_WORKSPACE_CONTROL_BYTES 262144

typedef enum {
    WKV_OK = 0,
    WKV_EINVAL = 1,       /* null/misaligned pointer, bad size, bad offsets, overlap */
    WKV_EUNSUPPORTED = 2, /* head size other than 64, unknown dtype */
    WKV_EWORKSPACE = 3,   /* workspace NULL or smaller than the query says */
    WKV_EHIP = 4          /* a HIP runtime call or kernel launch failed */
} wkv_status_t;

typedef enum {
    WKV_F32 = 0,
    WKV_BF16 = 1
} wkv_dtype_t;

/* Flags of wkv_prefill_ex / wkv_prefill_varlen_ex (bitwise OR; 0 = the plain
 * entry points' behaviour). */
typedef enum {
    /* The decay argument holds d_t instead of w_t, and w_t = exp(-exp(d_t))
     * (section 3.4, paragraph "Data-dependent decay").  Any d_t is legal:
     * -inf gives w = 1, +inf gives w = 0.  A bf16 d keeps the relative
     * precision of decays close to 1, which a bf16 w rounds to exactly 1. */
    WKV_FLAG_DECAY_LOG = 1,
    /* The Finch-C2 time mixer (section 3.4, paragraphs "Key computation with
     * normalization property", "Receptance, value, and the new second value"
     * and the output equation, per head, before LayerNorm and W_O):
     *   o_t[j]   = sum_i r_t[i] * S[i][j] + u2_t[j]
     *   S[i][j] <- w_t[i] * S[i][j] + k_t[i] * (1 - w_t[i]) * v_t[j]
     * i.e. k is the key projection BEFORE the (1 - w_t) factor, which the
     * library applies; there is no static bonus (u is ignored and may be
     * NULL); u2 = second_value is the data-dependent second value u'_t, or
     * NULL for none (the pages' ablation without it). */
    WKV_FLAG_FINCH_C2 = 2,
    /* o is written as bf16, each value rounded to nearest even from the fp32
     * result (the layout is unchanged: [.., H, D], 2 bytes per element).
     * state_out stays fp32.  Without the flag o is fp32. */
    WKV_FLAG_OUT_BF16 = 4
} wkv_flag_t;

/* FINCH_WKV_ABI_VERSION of the loaded library. */
int wkv_abi_version(void);

/* Static description of a status code (never NULL). */
const char *wkv_status_string(wkv_status_t status);

/* Detail of the last failed call on this thread ("" if none).  The pointer
 * stays valid until the next call into the library from the same thread. */
const char *wkv_last_error(void);

/*
 * Workspace size in bytes needed by wkv_prefill for these sizes (0 is a valid
 * answer: then workspace may be NULL).  Returns 0 as well for invalid sizes;
 * wkv_prefill reports those.  Deterministic: same arguments, same answer on the
 * same device.
 *
 * A nonzero workspace begins with WKV_WORKSPACE_CONTROL_BYTES of control
 * records: counters through which the workgroups of one launch hand
 * segment states to each other.  Zero its first WKV_WORKSPACE_CONTROL_BYTES
 * bytes once, before the first call that uses it (e.g. one hipMemset after
 * allocating it); every call leaves them ready for the next one, so they must
 * not be written between calls.  The rest of a workspace is scratch whose
 * contents do not matter.  A workspace sized for one call serves any call
 * whose query returns no more.
 */
size_t wkv_prefill_workspace_bytes(int B, int T, int H, int D, wkv_dtype_t in_dtype);

/*
 * Fixed-length batch pre-fill: B sequences of T tokens each.
 *   r, k, v, w  device, [B, T, H, D] of in_dtype, 16-byte aligned
 *   u           device, [H, D] fp32
 *   state_in    device, [B, H, D, D] fp32, or NULL (start from zeros)
 *   o           device, [B, T, H, D] fp32 (output; may be NULL only if T == 0)
 *   state_out   device, [B, H, D, D] fp32 (output), or NULL (not written)
 *   B >= 1, 1 <= H <= 65536, T >= 0, D == 64; sizes whose launch would exceed
 *   2^32 - 1 work-items in one grid dimension are rejected with
 *   WKV_EUNSUPPORTED (e.g. more than 2^24 - 1 (segment, head) work items)
 *   workspace   device scratch of at least wkv_prefill_workspace_bytes(...)
 *               bytes (NULL allowed when that is 0), 256-byte aligned
 *   stream      hipStream_t to enqueue on
 * T == 0 leaves o untouched and copies state_in (or zeros) to state_out.
 */
wkv_status_t wkv_prefill(const void *r, const void *k, const void *v,
                         const void *w, const float *u, const float *state_in,
                         float *o, float *state_out,
                         int B, int T, int H, int D, wkv_dtype_t in_dtype,
                         void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * Workspace size for wkv_prefill_varlen with these offsets (host copy).
 * Returns 0 for invalid offsets; wkv_prefill_varlen reports those.
 */
size_t wkv_prefill_varlen_workspace_bytes(const int32_t *cu_seqlens_host, int N,
                                          int H, int D, wkv_dtype_t in_dtype);

/*
 * Ragged (packed) pre-fill: N sequences concatenated along the token axis.
 *   cu_seqlens_dev   device, [N + 1] int32 token offsets
 *   cu_seqlens_host  host,   [N + 1] int32, the same values (used to plan the
 *                    launch; it must equal the device copy -- a mismatch gives
 *                    unspecified results but never an out-of-range access)
 *   Offsets: cu[0] == 0, non-decreasing, cu[N] = total tokens <= 2^31 - 1;
 *   empty sequences are allowed (their state is passed through).
 *   r, k, v, w, o    device, [cu[N], H, D]
 *   state_in/out     device, [N, H, D, D] fp32 (NULL as in wkv_prefill)
 * Each sequence starts from its own state_in[n] and ends in state_out[n].
 */
wkv_status_t wkv_prefill_varlen(const void *r, const void *k, const void *v,
                                const void *w, const float *u,
                                const int32_t *cu_seqlens_dev,
                                const int32_t *cu_seqlens_host, int N,
                                const float *state_in, float *o, float *state_out,
                                int H, int D, wkv_dtype_t in_dtype,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * Extended entry points: the plain ones with a flags word (wkv_flag_t) and
 * the Finch-C2 second value.
 *   decay         w_t, or d_t with WKV_FLAG_DECAY_LOG; same layout and type
 *                 as r
 *   u             [H, D] fp32 bonus; required unless WKV_FLAG_FINCH_C2 (then
 *                 ignored, may be NULL)
 *   second_value  with WKV_FLAG_FINCH_C2: u'_t, same layout and type as r, or
 *                 NULL (no second value); without the flag it must be NULL
 *   o             fp32, or bf16 with WKV_FLAG_OUT_BF16 (then [.., H, D] of
 *                 2-byte elements, 16-byte aligned)
 *   flags         unknown bits -> WKV_EUNSUPPORTED
 * Everything else (layouts, workspace size, aliasing, errors, T == 0, ragged
 * offsets) is exactly as for wkv_prefill / wkv_prefill_varlen, whose
 * workspace queries also size these calls.  wkv_prefill(...) is
 * wkv_prefill_ex(..., u, NULL, ..., flags = 0, ...).
 */
wkv_status_t wkv_prefill_ex(const void *r, const void *k, const void *v,
                            const void *decay, const float *u, const void *second_value,
                            const float *state_in, void *o, float *state_out,
                            int B, int T, int H, int D, wkv_dtype_t in_dtype,
                            unsigned flags, void *workspace, size_t workspace_bytes,
                            void *stream);

wkv_status_t wkv_prefill_varlen_ex(const void *r, const void *k, const void *v,
                                   const void *decay, const float *u,
                                   const void *second_value,
                                   const int32_t *cu_seqlens_dev,
                                   const int32_t *cu_seqlens_host, int N,
                                   const float *state_in, void *o, float *state_out,
                                   int H, int D, wkv_dtype_t in_dtype, unsigned flags,
                                   void *workspace, size_t workspace_bytes,
                                   void *stream);

/*
 * wkv_prefill_ex without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, results and validation as
 * wkv_prefill_ex; it allocates nothing.  Its scratch is a 36 MiB device array
 * inside the library that each GPU holds from the first such call until the
 * process ends (every fixed-length plan fits: at most about 34 MB are used).
 * All calls on one GPU share that array: calls that overlap in time on one
 * GPU (different streams, different threads without ordering) race and give
 * wrong results.  Calls ordered on one stream are safe.  The array starts
 * zeroed (static storage), which its control records need.
 */
wkv_status_t wkv_prefill_noalloc(const void *r, const void *k, const void *v,
                                 const void *decay, const float *u, const void *second_value,
                                 const float *state_in, void *o, float *state_out,
                                 int B, int T, int H, int D, wkv_dtype_t in_dtype,
                                 unsigned flags, void *stream);

/*
 * LayerNorm over the concatenated heads of each token: the normalisation of
 * the Finch-C2 output equation (section 3.4, output equation, applied to
 * r_t wkv_t + u'_t of all heads before W_O).  Per row of `width` values:
 *   y = (x - mean) / sqrt(var + eps) * gamma + beta
 * with the population mean and variance of the row.
 *   x          device, [tokens, width] fp32 (e.g. o of a pre-fill call seen as
 *              [tokens, H * D])
 *   gamma,beta device, [width] fp32
 *   y          device, [tokens, width] of out_dtype (WKV_BF16: round to
 *              nearest even; WKV_F32)
 *   width      multiple of 1024, at most 8192; eps finite, >= 0
 * 16-byte aligned pointers; y must not overlap an input.  Asynchronous on
 * `stream`; validation errors as for wkv_prefill.
 */
wkv_status_t wkv_layernorm_heads(const float *x, const float *gamma, const float *beta, float eps,
                                 void *y, wkv_dtype_t out_dtype, int64_t tokens, int width,
                                 void *stream);

/*
 * GOLD key compression c_t = x_t W_KD, d_model -> d_model / 16 (section "GOLD
 * Key Compression and TokenCat Decompression", compression step; x_t is the
 * output of the last Finch-C2 layer).
 *   x      device, [tokens, d_model] bf16
 *   w_kd   device, [d_model / 16, d_model] bf16: W_KD TRANSPOSED (the
 *          output-major layout of a linear layer's weight)
 *   c      device, [tokens, d_model / 16] of out_dtype (fp32, or bf16
 *          rounded to nearest even); fp32 accumulation
 *   d_model multiple of 1024, at most 65536; tokens <= 2^31 - 1
 * 16-byte aligned pointers; c must not overlap an input.
 */
wkv_status_t wkv_gold_compress(const void *x, const void *w_kd, void *c, wkv_dtype_t out_dtype,
                               int64_t tokens, int d_model, void *stream);

/*
 * Kernel timing hook for profiling tools (the benchmark uses it).  When
 * event_before/event_after (hipEvent_t, cast to void *) are non-NULL, every
 * later pre-fill call made from the calling thread attaches them to the launch
 * of its main scan kernel (the chunked kernel for bf16 -- for a split call in
 * one launch, that launch --, the token-serial one for fp32, the recurrent-step kernel when no sequence of the call has more
 * than 16 tokens; the one kernel of wkv_layernorm_heads and of
 * wkv_gold_compress): event_before takes that kernel's start timestamp and event_after
 * its end timestamp, so hipEventElapsedTime gives the kernel's own duration,
 * free of queue and launch gaps.  Pass NULL, NULL to stop.  The events are
 * owned by the caller, must be created with timing enabled and must outlive the
 * calls that record them.  Per thread; always returns WKV_OK.
 */
wkv_status_t wkv_set_kernel_timing_events(void *event_before, void *event_after);

/*
 * Launch form of split pre-fill calls, for comparisons and tests.  A bf16 call
 * that cuts its sequences into segments runs by default (launches = 1) as one
 * launch in which the segments' state pass, their combine and the chunked
 * scan hand results to each other through the workspace's control records;
 * it falls back to three launches (state pass, segment scan, chunked scan)
 * when the call has more than WKV_WORKSPACE_CONTROL_BYTES / 64 (sequence,
 * head) pairs or more state workgroups than the device holds at once.
 * launches = 3 always takes the three launches.  Both give identical results.
 * The one launch counts on its waiting workgroups being resident together
 * (the occupancy of an otherwise idle device): beside kernels of other
 * streams it may wait for them to leave, and a wait longer than about 1.3 s
 * ends the launch with that call's results void.  Callers that share the
 * device with long-running kernels should take the three launches.
 * Per thread; WKV_EINVAL for other values.
 */
wkv_status_t wkv_set_split_launches(int launches);

/*
 * Bound of each wait of the one launch (see wkv_set_split_launches), in ticks
 * of the GPU's 100 MHz clock, for tests of the error path: with a bound too
 * short for the workgroups to meet, waits expire, the launch still ends
 * normally, its results are void and wkv_workspace_errors reports it.  Per
 * thread; 0 restores the default of 2^27 ticks (about 1.3 s).  WKV_EINVAL
 * above 2^32 - 1.
 */
wkv_status_t wkv_set_wait_bound(unsigned long long ticks);

/*
 * Whether one-launch calls on a workspace kept their results.  A bounded wait
 * of the one launch (see wkv_set_split_launches) that expires marks its
 * (sequence, head) control record, and that call's results are void; the
 * mark stays until cleared here.  This reads the control records of
 * `workspace` (the first WKV_WORKSPACE_CONTROL_BYTES) after the work queued
 * on `stream` so far, waiting for that work, and sets *count to the number of
 * marked records (0: every one-launch call on the workspace since the marks
 * were last cleared kept its results).  With clear != 0 it then zeroes each
 * marked record whole: an expired wait can leave the record's counters out
 * of step, and later calls on the workspace may give wrong results without a
 * mark until it is cleared, so clear (or re-zero the control records) before
 * using a marked workspace again.  workspace NULL reads the static scratch of
 * wkv_prefill_noalloc on the current device (count 0 if no such call has
 * run there).  workspace_bytes 0 (a call that needed no workspace): count 0.
 *   WKV_EINVAL      count is NULL
 *   WKV_EWORKSPACE  0 < workspace_bytes < WKV_WORKSPACE_CONTROL_BYTES
 *   WKV_EHIP        the copy or the wait failed
 * Synchronous with the host (not for graph capture).
 */
wkv_status_t wkv_workspace_errors(const void *workspace, size_t workspace_bytes, int clear, int *count,
                                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FINCH_WKV_H */
