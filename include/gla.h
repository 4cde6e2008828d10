/*
 * gla.h - C ABI of the chunkwise gated linear attention forward for AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed (page "fla/ops/gla/fused_chunk.py": fused_chunk_gla and
 * FusedChunkGLAFunction.forward, with fused_chunk_gla_fwd_kernel for the
 * carried state and fwd_inner_chunk for the in-chunk term): for every
 * sequence n and head h a K x V fp32 state follows
 *
 *     S_t = diag(exp(g_t)) S_{t-1} + k_t v_t^T,     o_t = scale * q_t^T S_t,
 *
 * starting from S_0 = h0[n,h] (or 0) and ending at ht[n,h] = S_T.  It is
 * evaluated chunk by chunk (chunk = 64 tokens): in-chunk inclusive cumulative
 * log decay G, the causal (diagonal included) gated score term
 * (q exp(G)) (k exp(-G))^T v, and the inter-chunk term q exp(G) S with S
 * carried across chunks.  Packed variable-length batches follow page
 * "fla/ops/ttt/fused_chunk.py" (fused_chunk_ttt_linear): cu_seqlens holds
 * N+1 token offsets into a batch of one, the state restarts per sequence,
 * one h0 / ht per sequence.
 *
 * Conventions (all entry points):
 *  - Every pointer argument of gla_fwd is DEVICE memory owned by the caller;
 *    the library never allocates, frees or synchronises.  Work is enqueued on
 *    `stream` (a hipStream_t; NULL = the default stream) and runs
 *    asynchronously: results are valid once that stream has reached the call.
 *  - Layout is time-major and contiguous: q, k are [B, T, H, K], v and o are
 *    [B, T, HV, V], g is [B, T, HV, K] (a decay per key) or [B, T, HV] (one
 *    per value head and token), h0 and ht are [N, HV, K, V] (row-major, V
 *    fastest).  HV = H is the plain method; with HV a multiple of H, value head
 *    hv reads key head hv / (HV / H) (the head layout of page
 *    "fla/ops/gated_delta_rule/backends/triton_ascend/wy_fast.py",
 *    recompute_w_u_fwd_kernel_npu), and each value head has its own state.
 *  - Shapes: K and V are multiples of 16 in [16, 256]; any T >= 0, B >= 0,
 *    H >= 1.  Arguments are validated on the host before anything is
 *    enqueued; on any error nothing is written and the status says why.
 *  - cu_seqlens contents are a precondition (cu[0] = 0, non-decreasing,
 *    cu[N] = T) and are not checked.  Offsets that break it give undefined
 *    output values but no access outside the caller's buffers: the kernels
 *    clamp every sequence to [0, T) and never index past the workspace.
 *  - NaN / Inf inputs propagate; they are not checked.  g is a log decay
 *    (g <= 0, as logsigmoid gates are); any such finite gate is exact.  The
 *    chunk form's in-chunk factors exp(G_i - G_last) leave the fp32 range once
 *    a key decays by more than e^-80 within one 64-token chunk; a segment with
 *    such a chunk is evaluated again token by token by the same kernels (same
 *    results, slower).  Positive g makes the state grow and is only as exact as
 *    the fp32 range of the state allows.
 *  - Reentrant; the only global state is a per-device cache of the compute
 *    unit count.  Calls that share a workspace buffer must be ordered by the
 *    caller (same stream, or synchronised).
 */
#ifndef GLA_H_
#define GLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gla_status {
    GLA_OK = 0,
    GLA_ERR_NULL_ARG = 1,     /* a required pointer is NULL                      */
    GLA_ERR_BAD_SHAPE = 2,    /* negative / inconsistent sizes, B != 1 with cu_seqlens,
                                 or sizes whose index space exceeds the kernels' 32-bit grids */
    GLA_ERR_BAD_DTYPE = 3,    /* dtype is not GLA_F32 or GLA_BF16                */
    GLA_ERR_BAD_SCALE = 4,    /* scale is not finite and > 0                      */
    GLA_ERR_UNSUPPORTED = 5,  /* K, V, chunk or value_tile outside the supported set */
    GLA_ERR_WORKSPACE = 6,    /* workspace NULL or smaller than gla_fwd_workspace_bytes */
    GLA_ERR_HIP = 7           /* a HIP runtime call or kernel launch failed       */
} gla_status;

typedef enum gla_dtype {
    GLA_F32 = 0,   /* q, k, v, o are float32                                    */
    GLA_BF16 = 1   /* q, k, v, o are bfloat16; g, h0, ht are float32 either way */
} gla_dtype;

typedef enum gla_gate {
    GLA_GATE_PER_KEY = 0,   /* g [B, T, HV, K]: a log decay per key of the state */
    GLA_GATE_PER_HEAD = 1   /* g [B, T, HV]: one log decay per value head and token */
} gla_gate;

/* Bits of the status word (see gla_fwd's workspace). */
#define GLA_STATUS_WAIT_EXHAUSTED 1u  /* a bounded wait between waves ran out: the outputs may be wrong */

typedef struct gla_problem {
    int32_t B;        /* batch; must be 1 for packed sequences                         */
    int32_t T;        /* tokens per sequence, or total packed tokens with cu_seqlens  */
    int32_t H;        /* key heads (q, k)                                             */
    int32_t K;        /* key width: a multiple of 16 in [16, 256]                      */
    int32_t V;        /* value width: a multiple of 16 in [16, 256]                    */
    int32_t dtype;    /* gla_dtype of q, k, v and o                                   */
    int32_t n_seqs;   /* N: equal to B without cu_seqlens, len(cu_seqlens)-1 with it  */
    int32_t chunk;    /* chunk length in tokens; 64 is the supported value            */
    float scale;      /* multiplies q; finite and > 0 (callers map "default" to K^-0.5) */
    int32_t segment_chunks; /* 0: automatic.  Else chunks per state segment: a       */
                      /* sequence longer than this is split into segments whose start */
                      /* states are produced by a scan over segment summaries.        */
    int32_t packed;   /* 1 when cu_seqlens will be passed (packed sequences), else 0  */
    int32_t value_tile; /* 0: automatic.  Else value columns per workgroup, 64 or 128 */
                      /* (bf16 with K <= 128 only; a tuning choice, results agree)    */
    int32_t wait_limit; /* 0: default bound on each wait between waves (2^22 polls);  */
                      /* > 0: that many polls; -1: no polls, every such wait reports */
                      /* GLA_STATUS_WAIT_EXHAUSTED at once (a test hook)               */
    int32_t HV;       /* value heads (v, g, o, h0, ht): 0 means H; else a multiple of H */
    int32_t gate;     /* gla_gate: layout of g                                        */
    int32_t schedule; /* segmented sequences: 0 automatic (one pass for packed bf16  */
                      /* sequences, else three); 1 three passes (summaries, a scan of */
                      /* them, outputs); 2 one pass, segments chained by their end    */
                      /* states (bf16 with K <= 128, else three passes).  A tuning    */
                      /* choice: results agree to rounding.  gla_bwd: 0 automatic;    */
                      /* 1 a separate scan over the chunk summaries; 2 the scan       */
                      /* chained into the summary kernel; 3 the summary kernel walks  */
                      /* whole chains (gla_bwd only: gla_fwd rejects 3).  Results are */
                      /* the same.                                                    */
} gla_problem;

/*
 * Workspace bytes gla_fwd needs for problem `p` on the current device; at
 * least 256.  Returns (size_t)-1 when `p` is invalid.  The value depends on
 * the device's compute-unit count when segment_chunks is 0.
 */
size_t gla_fwd_workspace_bytes(const gla_problem *p);

/*
 * Chunkwise gated linear attention forward.
 *   q, k   : [B,T,H,K] dtype            g  : [B,T,HV,K] or [B,T,HV] float32, natural-log decay
 *   v      : [B,T,HV,V] dtype           h0 : [N,HV,K,V] float32 or NULL (zero state)
 *   cu_seqlens : [N+1] int32 token offsets or NULL (then N = B sequences of T tokens)
 *   o      : [B,T,HV,V] dtype, written for every token of every sequence
 *   ht     : [N,HV,K,V] float32 or NULL; when non-NULL it receives the state after
 *            each sequence's last token (h0, or zeros, for an empty sequence)
 *   workspace / workspace_bytes : device scratch of at least
 *            gla_fwd_workspace_bytes(p) bytes.  Its first 4 bytes are a sticky
 *            status word (uint32, GLA_STATUS_* bits): the kernels only ever set
 *            bits in it and the library never clears it, so the caller zeroes
 *            it once (for example when allocating the workspace) and reads it
 *            after the stream has reached the call.  The rest is scratch that
 *            each call overwrites.
 *   stream : hipStream_t to enqueue on
 * Returns GLA_OK or an error code (see gla_status); on error nothing is written.
 */
gla_status gla_fwd(const gla_problem *p,
                   const void *q, const void *k, const void *v, const float *g,
                   const float *h0, const int32_t *cu_seqlens,
                   void *o, float *ht,
                   void *workspace, size_t workspace_bytes,
                   void *stream);

/*
 * The same forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * instead of a caller workspace it uses a scratch array of 64 MiB that the
 * library holds on each device it runs on until the process ends, and it
 * calls no allocating routine.  Problems whose gla_fwd_workspace_bytes exceed
 * 64 MiB are rejected with GLA_ERR_WORKSPACE (the scratch holds the segment
 * summaries of long sequences and, for K > 128, the fp32 partial output
 * B*T*H*V*4 bytes).  Arguments and outputs are as for gla_fwd.
 *   status : a caller-owned device uint32 that receives the GLA_STATUS_* bits
 *            (OR-ed, never cleared: zero it first), or NULL to discard them.
 * Every call on one device shares that device's scratch: calls that overlap
 * in time on one device (different streams without ordering between them)
 * race and give undefined results; calls ordered on one stream are safe.
 * Returns GLA_OK or an error code; on error nothing is written.
 */
gla_status gla_fwd_noalloc(const gla_problem *p,
                           const void *q, const void *k, const void *v, const float *g,
                           const float *h0, const int32_t *cu_seqlens,
                           void *o, float *ht, uint32_t *status,
                           void *stream);

/*
 * Workspace bytes gla_bwd needs for problem `p` on the current device; at
 * least 256.  Returns (size_t)-1 when `p` is invalid for the backward.
 */
size_t gla_bwd_workspace_bytes(const gla_problem *p);

/*
 * Backward of the forward above (page "fla/ops/gla/fused_chunk.py":
 * FusedChunkGLAFunction.backward with fused_chunk_gla_bwd_kernel and
 * bwd_inner_chunk): for the loss L with dL/do = do_ and dL/dht = dht it returns
 * the gradients of q, k, v, g and h0.  With U_t = dL/dS_t of each sequence and
 * value head:
 *     dq_t = scale S_t do_t,  dk_t = U_t v_t,  dv_t = U_t^T k_t,
 *     dg_t = sum over tokens s >= t of (q_s * dq_s - k_s * dk_s)  +  rowsum(dht * ht)
 *     dh0  = dL/dS_0
 * (elementwise products; dq and dk of a key head sum over its value heads; a
 * per-head gate's gradient sums over keys).  Forward states are recomputed;
 * nothing from a forward call is needed.
 *   q, k, v, g, h0, cu_seqlens : as for gla_fwd (h0 NULL = zero state)
 *   do_    : [B,T,HV,V] dtype, gradient of o
 *   dht    : [N,HV,K,V] float32 gradient of ht, or NULL (zero)
 *   dq, dk : [B,T,H,K] dtype      dv : [B,T,HV,V] dtype
 *   dg     : [B,T,HV,K] float32 (per-key gate) or [B,T,HV] (per-head gate)
 *   dh0    : [N,HV,K,V] float32 or NULL (not computed)
 *   workspace / workspace_bytes : device scratch of at least
 *            gla_bwd_workspace_bytes(p) bytes, first 4 bytes a sticky status
 *            word as for gla_fwd (GLA_STATUS_WAIT_EXHAUSTED when a wait of the
 *            chained scan, see schedule, ran out).  It holds the state before
 *            every chunk and the state gradient reaching every chunk:
 *            2 * chunks * HV * K * min(V, 128) * 4 bytes and more.
 * Supported: K and V as for gla_fwd (K past 128 runs as two key blocks, whose
 * shares of dv are summed in fp32 before rounding; V past 128 as value slices
 * of 128 columns, whose shares of dq, dk and dg are summed the same way),
 * both dtypes, both gate layouts, HV a multiple of H, packed sequences.  Every
 * output row of a token is written; rows of other tokens are untouched.
 * Gates are exact as in the forward: a chunk in which some key decays by more
 * than e^-80 is evaluated token by token.  Returns GLA_OK or an error code; on
 * error nothing is written.  Pointers are device memory owned by the caller,
 * 16-byte aligned; work is asynchronous on `stream`.
 */
gla_status gla_bwd(const gla_problem *p,
                   const void *q, const void *k, const void *v, const float *g,
                   const float *h0, const int32_t *cu_seqlens,
                   const void *do_, const float *dht,
                   void *dq, void *dk, void *dv, float *dg, float *dh0,
                   void *workspace, size_t workspace_bytes,
                   void *stream);

/*
 * WY-representation forward of the gated delta rule, on the same chunk and
 * packed-sequence skeleton (page "fla/ops/gated_delta_rule/backends/
 * triton_ascend/wy_fast.py": recompute_w_u_fwd_kernel_npu and its wrapper
 * recompute_w_u_fwd_npu).  For every chunk of 64 tokens of a sequence
 * (restarting per packed sequence) and value head hv, with A_c the chunk's
 * 64 x 64 matrix:
 *     u = A_c (beta . v),    w = A_c (beta . 2^g . k)       (rows: the chunk's tokens)
 * k of key head hv / (HV / H); the factor 2^g (the page applies exp2 to g)
 * only when g is given.  A's columns past a partial chunk's tokens meet zero
 * rows and add nothing.
 */
typedef struct gla_wy_problem {
    int32_t B;        /* batch; 1 for packed sequences                        */
    int32_t T;        /* tokens per sequence, or total packed tokens          */
    int32_t H;        /* key heads (k)                                        */
    int32_t HV;       /* value heads (v, beta, A, g, w, u); a multiple of H; 0 means H */
    int32_t K;        /* key width, a multiple of 16 in [16, 256]             */
    int32_t V;        /* value width, a multiple of 16 in [16, 256]           */
    int32_t dtype;    /* gla_dtype of k, v, A, w and u; beta and g are float32 */
    int32_t n_seqs;   /* N: B without cu_seqlens, len(cu_seqlens)-1 with it   */
    int32_t chunk;    /* 64, the width of A's rows                           */
    int32_t packed;   /* 1 when cu_seqlens will be passed                     */
} gla_wy_problem;

/* Workspace bytes gla_wy_fwd needs (at least 256), or (size_t)-1 when invalid. */
size_t gla_wy_fwd_workspace_bytes(const gla_wy_problem *p);

/*
 *   k    : [B,T,H,K] dtype             v : [B,T,HV,V] dtype
 *   beta : [B,T,HV] float32            A : [B,T,HV,64] dtype, each token's row of its chunk matrix
 *   g    : [B,T,HV] float32 base-2 log gate, or NULL (no gate factor)
 *   cu_seqlens : [N+1] int32 or NULL
 *   w    : [B,T,HV,K] dtype            u : [B,T,HV,V] dtype (every token's row written)
 *   workspace / workspace_bytes : device scratch, first 4 bytes a status word as for gla_fwd
 * All pointers are device memory owned by the caller (16-byte aligned); work
 * is asynchronous on `stream`.  Returns GLA_OK or an error code; on error
 * nothing is written.
 */
gla_status gla_wy_fwd(const gla_wy_problem *p,
                      const void *k, const void *v, const float *beta, const void *A, const float *g,
                      const int32_t *cu_seqlens, void *w, void *u,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Static, human-readable name of a status code. */
const char *gla_status_str(gla_status s);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H_ */
