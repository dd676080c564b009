/*
 * sffn.h -- C ABI of the activation-sparse gated-FFN forward for MI355X (gfx950).
 *
 * The operation (one FFN layer, per token x of width d_model, d_ff channels):
 *
 *   z_i   = x . W_gate[i]                      gate pre-activation
 *           or (x . A) . B[:, i]               LoPA low-rank gate, rank r
 *   active = { i : z_i > tau }                 shifted-ReLU threshold, or
 *            the K channels of largest SiLU(z) per-token Top-K
 *   g_i   = z_i - tau   (threshold, LoPA)      gate value of an active channel
 *           SiLU(z_i)   (Top-K)
 *   y     = sum over active i of  g_i * (x . W_up[i]) * W_down[i]
 *
 * Sources: "Model Casting and Low-Parameter Gating: Towards More Sparsely
 * Activated FFNs" (paper detail page), Abstract -- compute the gating matrix's
 * output first and, because it is highly sparse, skip the two other matrices
 * for the zeroed channels; LoPA gating gives the gating matrix a low-FLOP,
 * low-parameter form. "Mixture-of-Channels: Exploiting Sparse FFNs for
 * Efficient LLMs Pre-Training and Inference" (blog summary), sections "Dentro il
 * 'mixture'" and "'Dentro MoC'" -- per token keep the Top-K channels of the
 * SwiGLU gate as a binary mask and, at inference, load only the weight rows and
 * columns of the active channels; the same summary ("Kernel e strutture")
 * names a 2:8 structured-sparsity option, read here as the top 2 of every
 * aligned group of 8 channels. "Model Casting ..." names top-p as a competing
 * sparsification and the PrunePath abstract activates units under a
 * cumulative-mass threshold on a softmax-normalised distribution: TOPP reads
 * these at channel granularity.
 *
 * Layout (all row-major, element type = the shape's dtype unless stated):
 *   x        [n_tokens][d_model]
 *   W_gate   [d_ff][d_model]   row i = channel i (this is nn.Linear(d, F).weight)
 *   W_up     [d_ff][d_model]   row i = channel i (nn.Linear(d, F).weight)
 *   W_down   [d_ff][d_model]   row i = channel i; the TRANSPOSE of
 *                              nn.Linear(F, d).weight, made contiguous once
 *   lopa_a   [rank][d_model]   A stored transposed (row k = column k of A)
 *   lopa_b   [d_ff][rank]      B stored transposed (row i = column i of B)
 *   y        [n_tokens][d_model] fp32, always
 *
 * Ownership: every pointer passed to sffn_forward is caller-owned device
 * memory that the library borrows for the duration of the work it enqueues on
 * `stream`; the library never allocates, copies or repacks. The workspace is
 * caller-allocated device memory of at least sffn_workspace_bytes(shape)
 * bytes, owned by the caller and used exclusively by one handle; a handle
 * must not run forwards on two streams at once. A handle holds only host-side
 * metadata. Nothing here is thread-safe per handle.
 *
 * Errors: every argument is validated on the host before anything is
 * enqueued; a failed check returns a negative status and enqueues nothing. A
 * failed kernel launch returns SFFN_ERR_HIP. Device faults surface at the
 * caller's next synchronisation. No C++ exception crosses this boundary.
 * sffn_forward never synchronises and never reads device memory on the host.
 */
#ifndef SFFN_H
#define SFFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SFFN_OK = 0,
    SFFN_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size, bad mode/k/n */
    SFFN_ERR_UNSUPPORTED = -2, /* a valid request the library does not implement */
    SFFN_ERR_HIP = -3,         /* a HIP runtime call or kernel launch failed */
    SFFN_ERR_WORKSPACE = -4    /* workspace null, misaligned or too small */
} sffn_status;

typedef enum { SFFN_F32 = 0, SFFN_BF16 = 1 } sffn_dtype;

typedef enum {
    SFFN_THRESHOLD = 0,  /* full gate; active = z > tau; g = z - tau            */
    SFFN_TOPK = 1,       /* full gate; active = per-token Top-K of SiLU(z); g = SiLU(z);
                            ties go to the lower channel index                   */
    SFFN_LOPA = 2,       /* low-rank gate (x.A).B; active = z > tau; g = z - tau  */
    SFFN_DENSE = 3,      /* full gate; every channel computed, g = max(z - tau, 0) */
    SFFN_DENSE_SILU = 4, /* full gate; every channel computed, g = SiLU(z) (SwiGLU) */
    SFFN_TOPK_2_8 = 5,   /* full gate; 2:8 structured: per token, within every aligned
                            group of 8 consecutive channels [8q, 8q + 8), the 2 of
                            largest SiLU(z) (ties to the lower index; a last group of
                            at most 2 channels keeps them all); g = SiLU(z)       */
    SFFN_TOPP = 6        /* full gate; top-p: per token, in the Top-K order of the keys
                            s = SiLU(z), the shortest prefix whose softmax mass
                            (exp(s_i) / sum_j exp(s_j)) reaches p, passed as tau,
                            0 < p <= 1; g = SiLU(z)                               */
} sffn_mode;

/* Shape of a layer and the largest batch a handle serves.
 *   d_model    > 0, multiple of 8
 *   d_ff       >= 1 (need not be a multiple of anything), at most 262144
 *   rank       0 for a full gate; otherwise the LoPA rank, a multiple of 8
 *   max_tokens >= 1; forwards take 0 <= n_tokens <= max_tokens
 *   dtype      SFFN_F32 or SFFN_BF16 (weights and x; y is fp32) */
typedef struct {
    int d_model;
    int d_ff;
    int rank;
    int max_tokens;
    int dtype;
} sffn_shape;

/* Device pointers to one layer's weights (layouts above). Each must be 16-byte
 * aligned. w_gate is required for THRESHOLD/TOPK/DENSE/DENSE_SILU, lopa_a and
 * lopa_b for LOPA; unused ones may be NULL. */
typedef struct {
    const void *w_gate;
    const void *lopa_a;
    const void *lopa_b;
    const void *w_up;
    const void *w_down;
} sffn_weights;

typedef struct sffn_ctx *sffn_handle;

/* Bytes of device workspace a handle with this shape needs; 0 if the shape is
 * invalid. Pure host arithmetic. */
size_t sffn_workspace_bytes(const sffn_shape *shape);

/* Create a handle. `workspace` is caller-owned device memory (256-byte
 * aligned, >= sffn_workspace_bytes(shape)); the library initialises it on the
 * first forward. Makes no HIP call. Returns SFFN_ERR_INVALID_ARG for a bad
 * shape or null `out`, SFFN_ERR_WORKSPACE for a bad workspace. */
sffn_status sffn_create(const sffn_shape *shape, void *workspace, size_t workspace_bytes,
                        sffn_handle *out);

/* One forward pass over n_tokens tokens, enqueued on `stream` (a hipStream_t;
 * NULL = the null stream).
 *   x           device, [n_tokens][d_model], shape dtype
 *   w           host struct of device weight pointers
 *   mode        an sffn_mode
 *   tau         threshold for THRESHOLD, LOPA and DENSE (compared in fp32); the
 *               mass p of TOPP, 0 < p <= 1
 *   k           Top-K size for TOPK, 1 <= k <= d_ff (ignored otherwise; TOPK_2_8
 *               keeps 2 of every 8 channels and takes no k)
 *   y           device, [n_tokens][d_model] fp32, written
 * Optional outputs (NULL to skip):
 *   active_idx  device int32 [n_tokens][d_ff]: row t holds token t's active
 *               channels in ascending order in its first active_cnt[t] slots
 *   active_cnt  device int32 [n_tokens]: active channels per token
 *   union_cnt   device int32 [1]: channels active for at least one token
 *   debug_z     device fp32 [n_tokens][d_ff]: the gate pre-activation z
 * A token with no active channel gets y = 0. n_tokens = 0 returns SFFN_OK and
 * enqueues nothing. LOPA needs a handle created with rank > 0; TOPK, TOPK_2_8,
 * TOPP, THRESHOLD and the dense modes need w_gate. */
sffn_status sffn_forward(sffn_handle handle, const void *x, int n_tokens, const sffn_weights *w,
                         int mode, float tau, int k, float *y, int32_t *active_idx,
                         int32_t *active_cnt, int32_t *union_cnt, float *debug_z, void *stream);

/* ---------------------------------------------------------------------------
 * Training: the forward with its activations stored in masked form, and the
 * backward over them. "Mixture-of-Channels" (blog summary), "Dentro il
 * 'mixture'": in training only the masked parts of the FFN activations are
 * kept for the backward, and the rest is rebuilt when the backward needs it.
 * Per token the stored rows hold the channels the mode keeps, ascending, with
 * their gate pre-activation z and up value u = x . W_up[i]; the backward
 * rebuilds g(z), g'(z) and h = g(z) u from them. With y as above and dy the
 * gradient of a loss with respect to y, over the stored channels:
 *   dh = dy . W_down[i],  du = dh g(z),  dz = dh u g'(z)
 *   dx = sum du W_up[i] + dz W_gate[i];  dW_down[i] += g(z) u dy,
 *   dW_up[i] += du x,  dW_gate[i] += dz x   (summed over tokens)
 * g' is 1 for THRESHOLD and DENSE (the shifted ReLU on its active branch;
 * DENSE stores only the channels with z > tau, the others carry no gradient)
 * and sigma(z) (1 + z (1 - sigma(z))) for the SiLU modes. The selection passes
 * no gradient. Both calls run the bf16 union path for any n_tokens (bf16
 * shapes only; LOPA is not supported: SFFN_ERR_UNSUPPORTED).
 * ------------------------------------------------------------------------- */

/* Stored activations, caller-owned device memory (4-byte aligned):
 *   cap   slots per token, 1 <= cap <= d_ff; at least k for TOPK, the 2:8
 *         count (2 per full group of 8, min(2, rest) for a last short group)
 *         for TOPK_2_8, d_ff for DENSE_SILU
 *   cnt   int32 [n_tokens]: channels the mode keeps for token t (written by
 *         the training forward); when it exceeds cap only the first cap are
 *         stored and the backward uses those
 *   idx   int32 [n_tokens][cap]: their channel indices, ascending
 *   z, u  fp32 [n_tokens][cap]: their gate pre-activation and up value */
typedef struct {
    int cap;
    int32_t *cnt;
    int32_t *idx;
    float *z;
    float *u;
} sffn_saved;

/* Bytes of the training workspace (caller-owned device memory, 256-byte
 * aligned) that sffn_forward_train and sffn_backward use for up to
 * shape->max_tokens tokens; 0 for an invalid shape. Pure host arithmetic. */
size_t sffn_train_workspace_bytes(const sffn_shape *shape);

/* A forward as sffn_forward (same x, w, mode, tau, k, y), always on the bf16
 * union path, that also writes the stored activations `saved`. Uses the
 * handle's workspace and train_ws (>= sffn_train_workspace_bytes). Errors as
 * sffn_forward, plus SFFN_ERR_INVALID_ARG for a bad `saved` and
 * SFFN_ERR_WORKSPACE for a bad train_ws. */
sffn_status sffn_forward_train(sffn_handle handle, const void *x, int n_tokens, const sffn_weights *w, int mode,
                               float tau, int k, float *y, const sffn_saved *saved, void *train_ws,
                               size_t train_ws_bytes, void *stream);

/* Backward over the stored activations of a training forward with the same
 * x, weights, mode, tau and k.
 *   dy       device, [n_tokens][d_model], bf16 (the shape's dtype)
 *   dx       device, [n_tokens][d_model] fp32, written
 *   dw_gate, dw_up, dw_down  device, [d_ff][d_model] fp32 (16-byte aligned),
 *            ADDED INTO: rows of channels no token stored are not touched;
 *            zero them before the first backward of an accumulation
 * x, dy, dx and the weight pointers 16-byte aligned. Uses train_ws (its
 * contents from the forward are not needed). Stored channel indices outside
 * [0, d_ff) are skipped. n_tokens = 0 returns SFFN_OK and enqueues nothing. */
sffn_status sffn_backward(sffn_handle handle, const void *x, const void *dy, int n_tokens, const sffn_weights *w,
                          int mode, float tau, int k, const sffn_saved *saved, float *dx, float *dw_gate,
                          float *dw_up, float *dw_down, void *train_ws, size_t train_ws_bytes, void *stream);

/* Token grouping for batches (opt-in; 1 = off, the default). With 2..8
 * groups, a forward of more than 8 tokens, at least 64 per group, and a
 * mode other than the dense ones groups its tokens by the channels they keep
 * and runs the up and down products of each group over the union of that
 * group's channels, instead of every token over the batch's union. SPT
 * abstract on the Hugging Face "Daily Papers" listing (query "FFN
 * modules"): a routed FFN batches tokens by the parameters they activate.
 * The grouping is k-means on the tokens' 0/1 channel masks (4 rounds,
 * seeded with evenly spaced tokens, deterministic). Outputs are the
 * forward's (a token's y uses only its own channels; sums may run in another
 * order). Such a forward SYNCHRONISES its stream once (the group sizes set
 * the launches), so it cannot be captured into a graph. Host-side only; no
 * HIP call here. SFFN_ERR_INVALID_ARG for groups outside 1..8. */
sffn_status sffn_set_token_groups(sffn_handle handle, int groups);

/* Bounded waits. The decode regime's down projection (1..8 tokens) sums its
 * channel groups inside one launch: the workgroup that sums a column slice
 * polls the other groups' partial sums, each tagged with the forward it
 * belongs to. It gives up after `polls` polls (default 262144; -1 gives up
 * at once, without polling, to exercise this path in tests), writes NaN to
 * the y entries it could not sum, and sets SFFN_ERR_BIT_DOWN_WAIT in the
 * sticky error word: the int32 at byte offset SFFN_WS_ERROR_OFFSET of the
 * workspace. The first forward on a handle zeroes that word; the library
 * never clears it afterwards (the caller may). A later forward is not
 * affected by a give-up. Host-side only; no HIP call here. */
#define SFFN_WS_ERROR_OFFSET 4
#define SFFN_ERR_BIT_DOWN_WAIT 1
sffn_status sffn_set_spin_limit(sffn_handle handle, int polls);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid it): sffn_forward for
 * one to 8 tokens (the decode regime) with no handle and no caller workspace.
 * Its workspace is a device array inside the library, SFFN_STATIC_SCRATCH_BYTES
 * bytes per GPU, held from the library's load until the process ends; the
 * first call on a GPU looks up that GPU's copy (hipGetSymbolAddress), and no
 * call allocates or frees anything.
 *   shape  as for sffn_create, with max_tokens <= 8; its workspace
 *          (sffn_workspace_bytes) must fit the array: SFFN_ERR_WORKSPACE
 *          otherwise, SFFN_ERR_UNSUPPORTED for max_tokens > 8
 *   other arguments, checks and results as sffn_forward, on the current device.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (two streams, or two host threads
 * with work in flight on different streams) race and give wrong results;
 * calls on one stream are ordered and safe. A call with a shape other than the
 * previous call's on that GPU first clears the array's control block and
 * slots. The sticky error word (sffn_set_spin_limit) sits at
 * SFFN_WS_ERROR_OFFSET of the array; the poll limit is the default. */
#define SFFN_STATIC_SCRATCH_BYTES (16u << 20)
sffn_status sffn_forward_noalloc(const sffn_shape *shape, const void *x, int n_tokens, const sffn_weights *w,
                                 int mode, float tau, int k, float *y, int32_t *active_idx, int32_t *active_cnt,
                                 int32_t *union_cnt, float *debug_z, void *stream);

/* Record two caller-created hipEvent_t (passed as void*) around the dominant
 * kernel of every later forward on this handle (the gate kernel, or the gate
 * GEMM on the batched path): ev_start before it, ev_stop after it, on the
 * forward's stream. Pass NULLs to stop. Host-side only; no HIP call here. */
sffn_status sffn_set_profile_events(sffn_handle handle, void *ev_start, void *ev_stop);

/* Release a handle (host metadata only; the workspace stays the caller's). */
sffn_status sffn_destroy(sffn_handle handle);

/* Static string naming a status code (never NULL). */
const char *sffn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SFFN_H */
