/*
 * rwkvwkv.h -- C ABI of librwkvwkv, the RWKV-4 WKV time-mixing path for AMD MI355X (gfx950).
 *
 * The operation (the WKV operator of the RWKV paper, arXiv 2305.13048, which the
 * "RWKV-4 14B" architecture page cites; the TR-2026-0009 port report describes it
 * in its Abstract, Methods and Reproducibility sections as a per-channel
 * numerator/denominator/max recurrence carried in fp32 with the max-trick,
 * followed by the receptance gate, with a token shift that mixes the current and
 * previous token):
 *
 *   per batch row b and channel c, with decay w_c (natural-log units, <= 0; the
 *   caller passes w = -exp(time_decay)) and bonus u_c,
 *
 *     wkv_t = ( e^{t w} N0 + sum_{i<t} e^{(t-1-i) w + k_i} v_i + e^{u + k_t} v_t )
 *           / ( e^{t w} D0 + sum_{i<t} e^{(t-1-i) w + k_i}     + e^{u + k_t}     )
 *
 *   where (N0, D0) = (aa e^pp, bb e^pp) is the prior state (zero when absent).
 *   Gated output: y_t = wkv_t / (1 + e^{-r_t}).
 *
 * State.  The recurrent state is a caller-owned, first-class object (the ChatRWKV
 * page, "The interesting bit" and Caveats: the caller tracks which text each
 * state belongs to).  It is planar fp32 [3][B][C] = (aa, bb, pp): numerator and
 * denominator scaled by e^{-pp}.  Triples are equivalence classes:
 * (aa, bb, pp) and (aa e^d, bb e^d, pp - d) are the same state; the library
 * returns some member of the class.  pp must be finite.  Pass state_in = NULL
 * for the empty state (no history).
 *
 * Layout.  Activations are row-major [B][T][C] (channel fastest, contiguous).
 * Per-channel parameters (w, u, mix_*) are fp32 [C].  All tensor pointers are
 * DEVICE memory owned by the caller; the library never frees them and holds no
 * pointer past the call (beyond stream ordering of the work it enqueued).
 *
 * Execution.  Every entry point only validates on the host and enqueues work on
 * `stream` (NULL = the null stream); it never synchronises.  All validation
 * happens before any work is enqueued, so an error return leaves every output
 * untouched.  Faults inside a kernel surface at the caller's next
 * synchronisation.  Nothing throws across the ABI.
 *
 * Errors.  Functions return RWKV_OK (0) or a negative rwkv_status;
 * rwkv_last_error() gives a thread-local message for the last failure.
 *
 * Sizes are int64; B, C >= 1 and T >= 0 (T = 0 copies the state).
 * Pointers must be aligned to their element size; when C % 4 == 0 and every
 * activation pointer is 8-byte (fp16) / 16-byte (fp32) aligned the kernels use
 * vector loads, otherwise a per-element path.  Inputs are assumed finite
 * (w may be -inf: full forgetting); NaN/Inf propagate unchecked.
 */
#ifndef RWKVWKV_H
#define RWKVWKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RWKV_ABI_VERSION 1

typedef enum rwkv_status {
    RWKV_OK = 0,
    RWKV_ERR_ARG = -1,    /* bad size, NULL required pointer, bad option, bad aliasing */
    RWKV_ERR_DTYPE = -2,  /* unknown dtype */
    RWKV_ERR_ALIGN = -3,  /* pointer not aligned to its element size */
    RWKV_ERR_HIP = -4,    /* the HIP runtime reported an error while enqueuing */
    RWKV_ERR_NOMEM = -5   /* the library-cached workspace could not be allocated */
} rwkv_status;

/* Element types of activations.  BF16 (bfloat16: fp32's exponent, 8 significand bits) is
   converted to fp32 on load and rounded to nearest-even on store, like F16; the recurrence
   and the state are always fp32. */
typedef enum rwkv_dtype { RWKV_F32 = 0, RWKV_F16 = 1, RWKV_BF16 = 2 } rwkv_dtype;

typedef enum rwkv_algo {
    RWKV_ALGO_AUTO = 0,        /* pick by shape: sequential for large B*C (or T <= 1), else
                                  chunked */
    RWKV_ALGO_SEQUENTIAL = 1,  /* one lane per (b, 4 channels), loop over T (large B*C) */
    RWKV_ALGO_CHUNKED = 2,     /* chunked scan over T in one launch: each tile gets its
                                  incoming state from its predecessors through a
                                  cross-workgroup look-back (long sequences) */
    RWKV_ALGO_TWO_PASS = 3     /* chunked scan in two launches: the aggregates of the tiles,
                                  then every tile folds its predecessors' aggregates (no waiting
                                  between workgroups; capturable; costs one more read of k, v) */
} rwkv_algo;

/*
 * How a single-launch chunked scan's tiles hand their states to the later tiles of their chain
 * (the workspace words of the look-back).  The GPU's eight XCDs each have their own L2, and
 * workgroups are dispatched to them round-robin by index.  When every workgroup is resident at
 * once and the workgroups of a time tile number a multiple of 8 (B * ceil(C / 64) chains, padded
 * with workgroups that return at once when that adds at most half again), all tiles of a chain
 * run on one XCD.
 */
typedef enum rwkv_publish {
    RWKV_PUBLISH_AUTO = 0,           /* L2_FIRST when the layout above holds (padding included),
                                        else WRITE_THROUGH */
    RWKV_PUBLISH_L2_FIRST = 1,       /* stored into the publishing XCD's L2 at once, where tiles
                                        on the same XCD read it without a trip to memory, and
                                        written through to memory after the tile's outputs: a
                                        tile on another XCD still sees it, only later */
    RWKV_PUBLISH_WRITE_THROUGH = 2   /* written through to memory at once */
} rwkv_publish;

/*
 * Options (all fields optional; pass NULL for: fp32 in and out, ungated, auto).
 * `size` must be set to sizeof(rwkv4_opts) (forward compatibility); the size of the struct
 * without its last field (`publish`, then taken as RWKV_PUBLISH_AUTO) is accepted too.
 */
typedef struct rwkv4_opts {
    uint32_t size;
    int32_t in_dtype;        /* rwkv_dtype of k, v, r (and x, x_prev, x_last, xk/xv_out) */
    int32_t out_dtype;       /* rwkv_dtype of y */
    const void *r;           /* rwkv4_wkv_forward only: [B,T,C] receptance, in_dtype;
                                NULL = ungated (y = wkv).  Must be NULL for timemix. */
    int32_t chunk_len;       /* chunked scan: tokens per workgroup tile; 0 = auto (128
                                for 2-byte inputs (fp16, bf16), 64 for fp32), else a power
                                of two in [16, 1024].  The single-launch scan stages a
                                tile's rows in LDS while they fit in 160 KB (2-byte inputs:
                                up to 512 tokens ungated, 256 gated or time mix; fp32:
                                half of those) and runs longer tiles as sub-tiles read
                                twice (aggregate, then output).  The two-pass scan stages
                                whole tiles only: RWKV_ERR_ARG above that limit. */
    int32_t algo;            /* rwkv_algo */
    void *workspace;         /* chunked scan scratch: NULL = library-cached per (device,
                                stream), allocated on first use;
                                else device memory of workspace_bytes >= the size
                                rwkv4_workspace_bytes() reports, zero-filled by the
                                caller once before its first use (RWKV_ALGO_CHUNKED
                                relies on it), then reusable */
    size_t workspace_bytes;
    int32_t publish;         /* rwkv_publish (RWKV_ALGO_CHUNKED only; results are identical
                                under every policy) */
} rwkv4_opts;

/*
 * WKV forward over a sequence (prefill).
 *   B, T, C      batch rows, tokens, channels.
 *   w, u         [C] fp32: decay (= -exp(time_decay), natural-log units) and bonus.
 *   k, v         [B,T,C] in_dtype.
 *   y            [B,T,C] out_dtype: wkv_t, or sigmoid(r_t) * wkv_t when opts->r is set.
 *   state_in     [3,B,C] fp32 prior state, or NULL for the empty state.
 *   state_out    [3,B,C] fp32 state after the T tokens, or NULL.  May equal
 *                state_in exactly (in-place update); no other overlap is allowed.
 * Workspace.  A chunked scan over more than one tile per chain needs scratch memory: the
 * caller's (opts->workspace) or, when that is NULL, a workspace the library allocates on first
 * use and keeps per (device, stream) until the process ends.  Calls on one stream may share a
 * workspace; calls that may run at the same time (different streams) must not, so a caller
 * that passes one workspace to several streams must serialise them itself.
 * Graph capture.  The single-launch chunked scan stamps its workspace per launch from the
 * host, so it cannot be replayed from a graph: on a capturing stream AUTO takes the two-pass
 * scan, which needs opts->workspace (RWKV_ERR_ARG without it), and RWKV_ALGO_CHUNKED, or a
 * chunk_len longer than the longest tile staged in LDS (which only the single-launch scan runs),
 * is refused with RWKV_ERR_ARG.  The sequential algorithm, and any call whose T fits in one
 * tile, capture as they are.
 * In the single-launch chunked scan a tile waits for the published states of earlier tiles
 * of its chain, which were dispatched before it, so the wait ends even when other kernels
 * share the GPU.  Each wait is still bounded (tens of milliseconds of polling): a wait that
 * gives up, which only a broken precondition (such as a workspace shared with a concurrent
 * call) can cause, writes NaN to its tile's outputs and sets the workspace's error word
 * instead of hanging the GPU.  While that word is set, every look-back on the workspace gives
 * up at once (its tiles' outputs are NaN), in the same call and in later ones, until
 * rwkv4_lookback_status reads and clears it.
 */
rwkv_status rwkv4_wkv_forward(int64_t B, int64_t T, int64_t C,
                              const float *w, const float *u,
                              const void *k, const void *v, void *y,
                              const float *state_in, float *state_out,
                              hipStream_t stream, const rwkv4_opts *opts);

/*
 * One decode token for B independent sequences (the T = 1 case of the forward,
 * with the state read and written in place).
 *   k, v         [B,C] in_dtype;  r [B,C] in_dtype or NULL (ungated).
 *   y            [B,C] out_dtype.
 *   state        [3,B,C] fp32, read and updated in place (required).
 */
rwkv_status rwkv4_wkv_step(int64_t B, int64_t C, const float *w, const float *u,
                           const void *k, const void *v, const void *r, void *y,
                           float *state, rwkv_dtype in_dtype, rwkv_dtype out_dtype,
                           hipStream_t stream);

/*
 * Time-mix core with the token shift and the receptance gate fused around the WKV
 * (the port report's "token-shift (mix current and previous token)" and
 * "time-mix gating").  With xs_0 = x_prev (zeros if NULL) and xs_t = x_{t-1}:
 *   xr = mix_r * x + (1 - mix_r) * xs   (fp32 math), receptance r := xr,
 *   y  = sigmoid(xr) * wkv(k, v)         with k, v supplied by the caller
 *                                        (its projections of xk, xv),
 *   xk_out = mix_k * x + (1 - mix_k) * xs,  xv_out likewise (each optional),
 *   x_last = x_{T-1} (the next call's x_prev; optional).
 *   x, k, v, xk_out, xv_out [B,T,C] and x_prev, x_last [B,C] use opts->in_dtype;
 *   y uses opts->out_dtype; mix_* [C] fp32.  State as in rwkv4_wkv_forward.
 */
rwkv_status rwkv4_timemix_fused(int64_t B, int64_t T, int64_t C,
                                const void *x, const void *x_prev, void *x_last,
                                const float *mix_k, const float *mix_v, const float *mix_r,
                                const void *k, const void *v,
                                const float *w, const float *u,
                                void *y, void *xk_out, void *xv_out,
                                const float *state_in, float *state_out,
                                hipStream_t stream, const rwkv4_opts *opts);

/*
 * rwkv4_timemix_fused for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments and results as
 * rwkv4_timemix_fused; it calls no hipMalloc or hipFree and no allocating routine.  Instead of a
 * workspace it uses a 16 MiB scratch array that the library holds in every GPU's memory until
 * the process ends (its address on a device is looked up on the first call there).  It runs the
 * sequential kernel (AUTO on large B*C, or RWKV_ALGO_SEQUENTIAL) or the two-pass scan, whose
 * launches neither wait for one another nor depend on the host, so calls may be captured; the
 * scratch holds the tile aggregates, 16 bytes per channel and tile, so a call may have at most
 * B * ceil(C / 64) * ceil(T / chunk_len) = 16384 tiles (B1 T65536 C2048 with 128-token
 * chunks; B1 T1024 C5120 needs 640), else RWKV_ERR_ARG.
 *   opts->workspace must be NULL and opts->algo must not be RWKV_ALGO_CHUNKED (RWKV_ERR_ARG);
 *   chunk_len is the two-pass scan's (at most 256 tokens for 2-byte inputs, 128 for fp32: the
 *   time mix stages three tensors of rows).
 * Every call on a GPU shares that GPU's scratch, and nothing in it needs clearing (each call
 * writes the aggregates it reads): calls that may run at the same time on one GPU (different
 * streams, or graphs replayed concurrently) race on it and must be serialised by the caller.
 */
rwkv_status rwkv4_timemix_fused_noalloc(int64_t B, int64_t T, int64_t C,
                                        const void *x, const void *x_prev, void *x_last,
                                        const float *mix_k, const float *mix_v, const float *mix_r,
                                        const void *k, const void *v,
                                        const float *w, const float *u,
                                        void *y, void *xk_out, void *xv_out,
                                        const float *state_in, float *state_out,
                                        hipStream_t stream, const rwkv4_opts *opts);

/*
 * Pre-LN token-shift prologue of either mixer (the "RWKV-4 14B" page, Facts table: a LayerNorm
 * before each mixer, ln1 before time mixing and ln2 before channel mixing; the port report's
 * Abstract: pre-LN and the token shift that mixes the current and previous token).  Per batch
 * row and token t, over the C channels of the row:
 *   n_t = (x_t - mean_t) / sqrt(var_t + ln_eps) * ln_weight + ln_bias
 *         (mean and biased variance of the row; n_t = x_t when ln_weight is NULL),
 *   xk_t = mix_k * n_t + (1 - mix_k) * n_{t-1}, and xv, xr likewise (fp32 math, one rounding),
 *   with n_{-1} = x_prev (the previous token's row, already normalised: a previous call's
 *   x_last; zeros when NULL), and x_last = n_{T-1} (x_prev, or zeros, when T = 0).
 * Time mixing asks for xk, xv, xr; channel mixing for xk, xr.
 *   x, xk, xv, xr [B,T,C] and x_prev, x_last [B,C] use dtype; ln_weight, ln_bias and the
 *   mixes are fp32 [C].  ln_bias may be NULL (zero) when ln_weight is set and must be NULL
 *   when it is not; ln_eps >= 0 and finite.  Each of xk, xv, xr is written exactly when its
 *   mix is given (both or neither when T > 0, else RWKV_ERR_ARG).  x_last may equal x_prev (the shift
 *   state updated in place); no other output may overlap an input or another output.
 */
rwkv_status rwkv4_shift_mix(int64_t B, int64_t T, int64_t C,
                            const void *x, const void *x_prev, void *x_last,
                            const float *ln_weight, const float *ln_bias, float ln_eps,
                            const float *mix_k, const float *mix_v, const float *mix_r,
                            void *xk, void *xv, void *xr,
                            rwkv_dtype dtype, hipStream_t stream);

/*
 * Receptance gate of channel mixing with the residual add (the port report's "channel-mix
 * gating"; the "RWKV-4 14B" page's field table: channel mixing has its own d x d receptance
 * matrix; the page's pre-norm placement puts the block's output on the residual stream):
 *   y = residual + kv / (1 + e^{-r})   elementwise over n values (residual NULL: 0),
 * where r and kv are the caller's projections (receptance, and value of the activated key).
 *   r, kv, residual: n values of in_dtype; y: n values of out_dtype.  y may be residual itself
 *   when the dtypes are equal (an in-place residual add); no other overlap.  n = 0 is a no-op.
 */
rwkv_status rwkv4_channelmix_gate(int64_t n, const void *r, const void *kv, const void *residual,
                                  void *y, rwkv_dtype in_dtype, rwkv_dtype out_dtype,
                                  hipStream_t stream);

/*
 * Whether a look-back wait of a single-launch chunked scan on a workspace gave up since the
 * workspace was zero-filled or last checked (the scans' outputs from then on hold NaN in every
 * tile that waited).  Safe to call at any time: it synchronises `stream` first, so the work
 * enqueued on it has finished, then reads the workspace's error word into *gave_up (1 set,
 * 0 clear) and clears it, so later calls on the workspace run normally again.
 *   workspace    the caller's workspace (opts->workspace of the calls), or NULL for the
 *                library-cached workspace of the current device and `stream` (*gave_up = 0
 *                when none exists yet).  The error word is the first 4 bytes of a workspace:
 *                a caller can set it to any nonzero value to make the next calls' look-backs
 *                give up at once, which exercises its own failure handling.
 *   stream       the stream whose work is waited for (and, with workspace NULL, whose cached
 *                workspace is read).
 * Returns RWKV_ERR_ARG for a NULL gave_up, RWKV_ERR_ALIGN for a workspace that is not 256-byte
 * aligned, RWKV_ERR_HIP if the synchronisation or the copy fails.
 */
rwkv_status rwkv4_lookback_status(void *workspace, hipStream_t stream, int32_t *gave_up);

/* Static text for a status code. */
const char *rwkv_status_string(rwkv_status s);

/* Thread-local message for the last non-OK return on this thread ("" if none). */
const char *rwkv_last_error(void);

/* Bytes of workspace the chunked scans need for this shape (chunk_len 0: enough for the
   automatic tile length of either input dtype). */
size_t rwkv4_workspace_bytes(int64_t B, int64_t T, int64_t C, int32_t chunk_len);

/* RWKV_ABI_VERSION of the loaded library. */
int rwkv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RWKVWKV_H */
