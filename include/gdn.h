/*
 * libgdn -- Gated DeltaNet chunked-prefill forward on AMD Instinct MI355X
 * (gfx950).  Plain C ABI: no C++ or framework types cross it.
 *
 * The operation (FlashQLA pages, aisparkup.com wiki "high-level API" and
 * "low-level API"; agentlenshq.com blog "GDN chunked-prefill optimisation"):
 * for every sequence n and value head j, with key/query head
 * i = j / (H_v / H_qk), run the gated delta rule
 *
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t
 *
 * from S_0 = initial_state (or zero) and return o and the final state.  The
 * library evaluates it chunk by chunk (chunks of 64 tokens, WY form), with
 * optional intra-GPU context parallelism (AutoCP, blog section "gate-driven
 * automatic intra-card context parallelism": the chunk axis of a sequence is
 * cut into segments of L chunks; a segment either starts from a state rebuilt
 * by a short warm-up over the preceding chunks, whose influence decays with
 * the gates, or from the exact state given by per-segment transition maps).
 *
 * Conventions for every entry point
 *   - All tensors are dense, row-major, in device memory unless a field says
 *     host.  Layouts (element types in brackets):
 *        q, k   [B, T, H_qk, K]  (bf16)     v      [B, T, H_v, V] (bf16)
 *        g, beta [B, T, H_v]      (fp32)     o      [B, T, H_v, V] (bf16 or fp32)
 *        initial_state, final_state [N, H_v, K, V] (fp32), stored as S^T
 *        cu_seqlens [N + 1] (int32): packed sequences, B must be 1
 *   - The caller owns every buffer, including the workspace; the library
 *     never allocates, frees or synchronises.  Work is enqueued on `stream`
 *     (a hipStream_t; NULL = the null stream) and runs asynchronously.
 *   - Inputs are read-only.  o must not overlap any input; final_state must
 *     not overlap initial_state or any other tensor.
 *   - q, k, v and o must be 16-byte aligned, g and beta 4-byte aligned.
 *   - One chunk (64 token rows) of every tensor must span less than 2 GiB
 *     (64 * max(H_qk * K * 2, H_v * V * sizeof(o element), H_v * 64 * 4) bytes
 *     < 2^31), otherwise GDN_EUNSUPPORTED.  Sequence length is not limited.
 *   - Return value: GDN_OK (0) or a negative gdn_status.  Arguments are fully
 *     validated before anything is enqueued, so a failed call launches
 *     nothing.  gdn_last_error() gives a message for the calling thread's
 *     last failure.  No exception crosses the ABI.
 *   - NaN/Inf inputs propagate; they are not trapped.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 4

typedef enum {
    GDN_OK = 0,
    GDN_EINVAL = -1,        /* bad shape, pointer, offsets or aliasing */
    GDN_EUNSUPPORTED = -2,  /* valid request this library does not implement (K, V, chunk) */
    GDN_EWORKSPACE = -3,    /* workspace missing or smaller than gdn_fwd_plan asked for */
    GDN_EHIP = -4           /* a HIP launch or query failed; message has the HIP text */
} gdn_status;

typedef enum { GDN_DTYPE_BF16 = 0, GDN_DTYPE_F32 = 1 } gdn_dtype;

/* Intra-GPU context parallelism over the chunk axis.
 *   OFF    one workgroup per (sequence, v-head) runs every chunk in order.
 *   WARMUP segments of L chunks; a segment not at its sequence start first
 *          runs the state pass (no output) from a zero state over the chunks
 *          before it, as many as it takes for the summed log-gates of the
 *          window to reach ln(2^-24) (the fp32 noise floor), or back to the
 *          sequence start, where the walk begins from initial_state and is
 *          exact.  The state error a window leaves is at most exp(sum of its
 *          log-gates) times the state norm at its far end (unit keys, beta in
 *          [0, 2]), so it sits below fp32 resolution whatever the gates; weak
 *          gates only make the windows (and the call) longer.  A positive
 *          cp_warmup_chunks caps the window, and then that bound, not fp32
 *          resolution, is the error guarantee.
 *   EXACT  segments of L chunks; a pre-pass computes each segment's
 *          zero-start state S and transition map M, a combine pass chains
 *          H <- M H + S across segments, and the main pass starts every
 *          segment from its exact state.
 *   AUTO   WARMUP with L chosen from the occupancy of the GPU (OFF when one
 *          segment per sequence fills it). */
typedef enum { GDN_CP_OFF = 0, GDN_CP_EXACT = 1, GDN_CP_WARMUP = 2, GDN_CP_AUTO = 3 } gdn_cp_mode;

typedef struct {
    int64_t B;                  /* batch rows (1 when cu_seqlens is used) */
    int64_t T;                  /* tokens per row (total packed tokens when varlen) */
    int32_t H_qk, H_v;          /* key/query heads, value heads; H_v % H_qk == 0 */
    int32_t K, V;               /* head dims; this library supports K = V = 128 */
    int32_t num_seqs;           /* N: B, or len(cu_seqlens) - 1 when varlen */
    const int32_t *cu_seqlens_host; /* host copy of the offsets, required for varlen planning; NULL otherwise */
    float scale;                /* output scale (callers usually pass K^-1/2) */
    int32_t has_h0;             /* initial_state given */
    int32_t want_ht;            /* final_state requested */
    int32_t o_dtype;            /* gdn_dtype of o */
    int32_t chunk;              /* chunk length; must be 64 */
    int32_t cp_mode;            /* gdn_cp_mode */
    float cp_lambda;            /* >0: segment length L = round(lambda * sqrt(chunks of the longest sequence)) */
    int32_t cp_segment_chunks;  /* >0: fixed L (overrides cp_lambda and AUTO) */
    int32_t cp_warmup_chunks;   /* WARMUP/AUTO window cap in chunks; <= 0: no cap (gate-driven window) */
} gdn_fwd_desc;

typedef struct {
    size_t workspace_bytes;     /* bytes gdn_fwd needs at `workspace` (256-byte aligned) */
    int32_t total_chunks;       /* sum over sequences of ceil(len / chunk) */
    int32_t segment_chunks;     /* L actually used (= longest sequence's chunk count when CP is off) */
    int32_t num_segments;       /* segments over all sequences (per v-head) */
    int32_t warmup_chunks;      /* window cap used by WARMUP/AUTO; 0: none, or CP off */
    int32_t cp_mode;            /* resolved mode (AUTO becomes WARMUP or OFF) */
    int32_t workgroups;         /* main-kernel workgroups = num_segments * H_v */
} gdn_fwd_plan_info;

typedef struct {
    const void *q, *k, *v;          /* bf16 */
    const float *g, *beta;          /* fp32 */
    const float *initial_state;     /* fp32, NULL iff has_h0 == 0 */
    const int32_t *cu_seqlens;      /* device offsets, NULL iff the call is not varlen */
    void *o;                        /* bf16 or fp32 per o_dtype */
    float *final_state;             /* fp32, NULL iff want_ht == 0 */
    /* Low-level outputs (wiki, "low-level API": g, A, o, h, final_state),
     * optional (NULL = not produced), 16-byte aligned, caller-owned, and not
     * overlapping any other tensor:
     *   h  fp32 [total_chunks, H_v, K, V]: S^T at the start of every chunk,
     *      chunks of all sequences in order (total_chunks from gdn_fwd_plan);
     *   A  fp32 [B * T, H_v, chunk]: for the token in row i of its chunk, row
     *      i of that chunk's WY matrix (I + A~)^{-1}, A~_is = beta_i
     *      exp(G_i - G_s) k_i.k_s for s < i (unit diagonal, zeros above it).
     * With WARMUP/AUTO context parallelism, h at a segment's chunks carries
     * the warm-up approximation of the state (the same as o); h of a chunk
     * that is only a warm-up chunk of a later segment is written by the
     * segment that owns it.
     *   v_new fp32 [total_chunks, H_v, chunk, V]: v' = U - W h of every chunk
     *      (the delta-rule residuals of the chunked form), all `chunk` rows,
     *      zero past a sequence's end; kept for gdn_bwd. */
    float *h;
    float *A;
    float *v_new;
} gdn_fwd_ptrs;

/* ABI version this library was built with (GDN_ABI_VERSION). */
int gdn_abi_version(void);

/* Static text for a gdn_status value. */
const char *gdn_status_str(int status);

/* Message for the calling thread's most recent failure ("" if none). */
const char *gdn_last_error(void);

/* Host-only planning: validates the descriptor (shapes, offsets, support),
 * resolves the context-parallel layout and sizes the workspace.  Makes no HIP
 * call, so it works without a GPU.  `out` may be NULL (validation only). */
int gdn_fwd_plan(const gdn_fwd_desc *d, gdn_fwd_plan_info *out);

/* Forward pass: o and (optionally) final_state from the inputs in `p`.
 * Re-plans `d` (same validation as gdn_fwd_plan), checks pointers and
 * aliasing, then enqueues the kernels on `stream`.  `workspace` must hold at
 * least gdn_fwd_plan's workspace_bytes and be 256-byte aligned; it may be NULL
 * when that size is 0 (CP modes OFF, WARMUP and AUTO keep all intermediates
 * on chip).  Its contents on entry do not matter and are scratch afterwards. */
int gdn_fwd(const gdn_fwd_desc *d, const gdn_fwd_ptrs *p, void *workspace, size_t workspace_bytes,
            void *stream);

/* Forward pass that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, validation, kernels and results as
 * gdn_fwd, without the workspace arguments: the workspace gdn_fwd_plan sizes
 * (non-zero only for GDN_CP_EXACT: per-segment S, M and start states) lives in
 * a static device array of GDN_NOALLOC_SCRATCH_BYTES owned by the library, one
 * per GPU, held from the library's load until the process ends.  The caller
 * still passes every input and output.
 *   - A call whose plan needs more than GDN_NOALLOC_SCRATCH_BYTES returns
 *     GDN_EWORKSPACE and launches nothing.
 *   - The calling thread's current device must be the device `stream` belongs
 *     to (GDN_EINVAL otherwise).
 *   - Every call on one GPU shares that GPU's array: calls that may overlap in
 *     time on one GPU (different streams, or host threads) race and must be
 *     serialised by the caller.  Nothing in the array needs to start at zero
 *     (every word a call reads was written earlier in the same call).
 *   - Calls no hipMalloc, hipFree or other allocating routine. */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)
int gdn_fwd_noalloc(const gdn_fwd_desc *d, const gdn_fwd_ptrs *p, void *stream);

/* Chunk-local running sum of the log-gates (the transformed g returned by the
 * pages' low-level forward, aisparkup.com wiki "low-level API"):
 * out[t] = sum of g over the tokens of t's chunk up to and including t.
 * Chunks of `chunk` tokens start at every sequence start.
 * g, out: fp32 [B, T, H] device; cu_seqlens: device int32 [num_seqs + 1] or
 * NULL (then num_seqs must equal B).  out may equal g (in place). */
int gdn_chunk_cumsum(const float *g, float *out, int64_t B, int64_t T, int32_t H, int32_t chunk,
                     const int32_t *cu_seqlens, int32_t num_seqs, void *stream);

/* ------------------------------------------------------------------ backward
 *
 * The chunked backward the pages announce (agentlenshq.com blog, title and
 * "performance benchmarks"; aisparkup.com wiki, "key features": a fused
 * backward alongside the forward): the gradients of a scalar loss with
 * respect to q, k, v, g, beta and initial_state, given dO = dL/do and
 * optionally dL/d final_state.  The result is the exact derivative of the
 * forward above, evaluated chunk by chunk: a reverse pass over the chunks
 * (the adjoint of the state pass) followed by independent per-chunk
 * gradients.  Gradients flow through every input; dq and dk of a key/query
 * head sum the contributions of the value heads that share it; dg is the
 * gradient with respect to the per-token log-gates (not their cumsum).
 *
 * Context parallelism of the reverse pass, with the forward's segment rule:
 * OFF; WARMUP / AUTO, a segment that does not end its sequence starts from zero
 * after a warm-up over the chunks that follow it (the forward's gate window:
 * the state gradient decays with the same gates); EXACT, a pre-pass computes
 * each segment's zero-start result and transition map (K x K), a combine pass
 * chains them from the sequence end, and every segment starts from its exact
 * gradient.
 */
typedef struct {
    gdn_fwd_desc fwd;     /* the forward call being differentiated (want_ht and o_dtype are ignored) */
    int32_t has_dht;      /* d_final_state given */
    int32_t grad_dtype;   /* gdn_dtype of dq, dk, dv (dg, dbeta, d_initial_state are fp32) */
    int32_t saved_fwd;    /* 1: the caller passes h, A and v_new from gdn_fwd under the same fwd
                             descriptor; 0: the backward recomputes them in its workspace */
} gdn_bwd_desc;

typedef struct {
    size_t workspace_bytes;     /* bytes gdn_bwd needs at `workspace` (256-byte aligned) */
    int32_t total_chunks;
    int32_t segment_chunks;     /* L of the reverse pass */
    int32_t num_segments;       /* reverse-pass segments over all sequences (per v-head) */
    int32_t warmup_chunks;      /* window cap of the reverse pass; 0: none, or CP off */
    int32_t cp_mode;            /* resolved mode of the reverse pass (OFF, EXACT or WARMUP) */
    int32_t workgroups_reverse; /* reverse-pass workgroups = num_segments * H_v * 2 */
    int32_t workgroups_local;   /* per-chunk workgroups = (total_chunks + empty sequences) * H_qk */
} gdn_bwd_plan_info;

typedef struct {
    const void *q, *k, *v;          /* bf16, as for gdn_fwd */
    const float *g, *beta;          /* fp32 */
    const float *initial_state;     /* fp32, NULL iff fwd.has_h0 == 0 */
    const int32_t *cu_seqlens;      /* device offsets, NULL iff not varlen */
    const void *dO;                 /* bf16 [B, T, H_v, V] */
    const float *d_final_state;     /* fp32 [N, H_v, K, V], NULL iff has_dht == 0 */
    const float *h;                 /* saved_fwd: gdn_fwd's h (fp32 [total_chunks, H_v, K, V]), else NULL */
    const float *A;                 /* saved_fwd: gdn_fwd's A (fp32 [B * T, H_v, chunk]), else NULL */
    const float *v_new;             /* saved_fwd: gdn_fwd's v_new (fp32 [total_chunks, H_v, chunk, V]), else NULL */
    void *dq, *dk;                  /* [B, T, H_qk, K], grad_dtype */
    void *dv;                       /* [B, T, H_v, V], grad_dtype */
    float *dg, *dbeta;              /* fp32 [B, T, H_v] */
    float *d_initial_state;         /* fp32 [N, H_v, K, V], or NULL (not written) */
} gdn_bwd_ptrs;

/* Host-only planning of the backward: validates (as gdn_fwd_plan, plus the
 * backward's own fields), resolves the reverse pass's CP layout and sizes the
 * workspace.  No HIP call.  `out` may be NULL. */
int gdn_bwd_plan(const gdn_bwd_desc *d, gdn_bwd_plan_info *out);

/* Backward pass.  Same conventions as gdn_fwd: caller-owned buffers, inputs
 * read-only, outputs must not overlap inputs or each other, full validation
 * before anything is enqueued, asynchronous on `stream`.  dq, dk, dv, dO
 * 16-byte aligned; g, beta, dg, dbeta 4-byte aligned; state tensors, h and A
 * 16-byte aligned.  Every element of dq, dk, dv, dg and dbeta is written. */
int gdn_bwd(const gdn_bwd_desc *d, const gdn_bwd_ptrs *p, void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
