/*
 * CPU oracle for the chunkwise gated linear attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no source with the GPU library.
 *
 * What it computes is the plain definition of the method, not the chunked
 * algorithm: for every sequence n and head h it runs the gated linear
 * attention recurrence token by token in double precision,
 *
 *     S_0 = h0[n,h]  (or 0)                     S is a K x V matrix
 *     S_t = diag(exp(g_t)) S_{t-1} + k_t v_t^T   (decay first, then add)
 *     o_t = scale * q_t^T S_t                    (the updated state)
 *     ht[n,h] = S_T
 *
 * Sources (page "fla/ops/gla/fused_chunk.py"):
 *   - fused_chunk_gla_fwd_kernel: the state is decayed row-wise by exp of the
 *     chunk's log decay and then receives k^T v; h0 enters before the first
 *     chunk and ht is the state after the last one, kept in fp32.
 *   - prepare_qg_kg and fwd_inner_chunk: within a chunk, with G the inclusive
 *     cumulative sum of g, the query is weighted by exp(G_i), a key entering
 *     the carried state by exp(G_last - G_j), and the in-chunk score of key j
 *     for query i by exp(G_i - G_j) under a causal mask that keeps j <= i
 *     (diagonal included).  These weights make the chunked form equal, term
 *     by term, to the token recurrence above with the output read after the
 *     update.
 *   - FusedChunkGLAFunction.forward: g is a natural-log decay (exp, not exp2).
 * Packed variable-length sequences follow the page "fla/ops/ttt/fused_chunk.py"
 * (fused_chunk_ttt_linear_fwd_kernel and fused_chunk_ttt_linear): sequence n
 * owns tokens [cu[n], cu[n+1]) of a batch of one, the state restarts per
 * sequence, and there is one initial / final state per sequence.
 *
 * Precision: q, k, v, g are read as float32 (bf16 inputs are handed over
 * upcast, which is exact) and promoted to double, h0 is double; all arithmetic is double,
 * exp is the C library's.  Build: gcc -O2 -fopenmp -shared -fPIC, no fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * Head and gate variants (page "fla/ops/gated_delta_rule/backends/triton_ascend/wy_fast.py",
 * recompute_w_u_fwd_kernel_npu and its wrapper): keys and queries have H heads,
 * values, gates and states have HV heads (HV a multiple of H), and value head hv
 * reads key / query head hv / (HV / H).  The gate is either one log decay per
 * key (g [T][HV][K]) or one per value head and token (g [T][HV], the same decay
 * for every key of the state).
 *
 * q, k    : [T_total][H][K] float32, time-major (token, head, key)
 * v       : [T_total][HV][V] float32
 * g       : [T_total][HV][K] float32 (gate_per_head = 0) or [T_total][HV] (= 1)
 * offsets : [N+1] int64 token offsets, offsets[0] = 0, non-decreasing
 * h0      : [N][HV][K][V] double or NULL (zero initial state); double so that a
 *           final state can be fed back unrounded (fp32 h0 upcasts exactly)
 * o       : [T_total][HV][V] double, every token of every sequence is written
 * ht      : [N][HV][K][V] double or NULL
 * nthreads: OpenMP threads to use (<= 0: library default)
 * Returns 0, or -1 on invalid sizes / allocation failure (nothing written).
 */
int gla_oracle_fwd_heads(int64_t N, const int64_t *offsets, int64_t H, int64_t HV, int64_t K, int64_t V,
                         int gate_per_head, const float *q, const float *k, const float *v, const float *g,
                         const double *h0, double scale, double *o, double *ht, int nthreads)
{
    if (N < 0 || H <= 0 || HV <= 0 || HV % H != 0 || K <= 0 || V <= 0 || !offsets || !o)
        return -1;
    for (int64_t n = 0; n < N; ++n)
        if (offsets[n + 1] < offsets[n]) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int64_t group = HV / H;
    int failed = 0;
    const int64_t jobs = N * HV;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t job = 0; job < jobs; ++job) {
        const int64_t n = job / HV, hv = job % HV, hk = hv / group;
        double *S = (double *)malloc(sizeof(double) * (size_t)(K * V));
        double *acc = (double *)malloc(sizeof(double) * (size_t)V);
        if (!S || !acc) { free(S); free(acc); failed |= 1; continue; }
        if (h0) {
            memcpy(S, h0 + (n * HV + hv) * K * V, sizeof(double) * (size_t)(K * V));
        } else {
            memset(S, 0, sizeof(double) * (size_t)(K * V));
        }
        for (int64_t t = offsets[n]; t < offsets[n + 1]; ++t) {
            const float *qt = q + (t * H + hk) * K;
            const float *kt = k + (t * H + hk) * K;
            const float *vt = v + (t * HV + hv) * V;
            for (int64_t j = 0; j < V; ++j) acc[j] = 0.0;
            for (int64_t i = 0; i < K; ++i) {
                const float gi = gate_per_head ? g[t * HV + hv] : g[(t * HV + hv) * K + i];
                const double decay = exp((double)gi);
                const double ki = (double)kt[i];
                const double qi = (double)qt[i];
                double *row = S + i * V;
                for (int64_t j = 0; j < V; ++j) {
                    row[j] = decay * row[j] + ki * (double)vt[j];
                    acc[j] += qi * row[j];
                }
            }
            double *ot = o + (t * HV + hv) * V;
            for (int64_t j = 0; j < V; ++j) ot[j] = scale * acc[j];
        }
        if (ht) memcpy(ht + (n * HV + hv) * K * V, S, sizeof(double) * (size_t)(K * V));
        free(S);
        free(acc);
    }
    return failed ? -1 : 0;
}

/* The method with one value head per key head and a decay per key (HV = H). */
int gla_oracle_fwd(int64_t N, const int64_t *offsets, int64_t H, int64_t K, int64_t V,
                   const float *q, const float *k, const float *v, const float *g,
                   const double *h0, double scale, double *o, double *ht, int nthreads)
{
    return gla_oracle_fwd_heads(N, offsets, H, H, K, V, 0, q, k, v, g, h0, scale, o, ht, nthreads);
}

/*
 * Backward of the recurrence (the gradients that page "fla/ops/gla/fused_chunk.py"
 * computes in FusedChunkGLAFunction.backward, fused_chunk_gla_bwd_kernel,
 * bwd_inner_chunk and bwd_decay_global_cumsum, here by the chain rule of the
 * token recurrence itself), for one value head per key head and a decay per key.
 * With L = sum_t do_t . o_t + <dht, S_T>, and U_t = dL/dS_t (all later uses):
 *
 *     U_T = dht + scale q_T do_T^T,   U_t = diag(exp(g_{t+1})) U_{t+1} + scale q_t do_t^T
 *     dq_t = scale S_t do_t           dk_t = U_t v_t           dv_t = U_t^T k_t
 *     dg_t = exp(g_t) * rowsum(U_t (.) S_{t-1})               dh0 = diag(exp(g_1)) U_1
 *
 * (S_{t-1} of the first token is h0.)  The page's backward takes no dht and
 * returns no dh0; here dht may be given (NULL: zero) and dh0 is returned when
 * asked for.  Every S_t of a (sequence, head) is kept, so memory is
 * T * K * V doubles per job (test sizes only).
 *
 * Arguments as gla_oracle_fwd plus: do_ [T][H][V], dht [N][H][K][V] double or NULL;
 * outputs dq, dk [T][H][K], dv [T][H][V], dg [T][H][K], dh0 [N][H][K][V] or NULL,
 * all double.
 */
int gla_oracle_bwd(int64_t N, const int64_t *offsets, int64_t H, int64_t K, int64_t V,
                   const float *q, const float *k, const float *v, const float *g,
                   const double *h0, double scale, const float *do_, const double *dht,
                   double *dq, double *dk, double *dv, double *dg, double *dh0, int nthreads)
{
    if (N < 0 || H <= 0 || K <= 0 || V <= 0 || !offsets || !dq || !dk || !dv || !dg)
        return -1;
    for (int64_t n = 0; n < N; ++n)
        if (offsets[n + 1] < offsets[n]) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int failed = 0;
    const int64_t jobs = N * H;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t job = 0; job < jobs; ++job) {
        const int64_t n = job / H, h = job % H;
        const int64_t t0 = offsets[n], L = offsets[n + 1] - offsets[n];
        const int64_t KV = K * V;
        /* states S_{-1} (h0) .. S_{L-1}, one K x V block each */
        double *S = (double *)malloc(sizeof(double) * (size_t)((L + 1) * KV));
        double *U = (double *)malloc(sizeof(double) * (size_t)KV);
        if (!S || !U) { free(S); free(U); failed |= 1; continue; }
        if (h0) memcpy(S, h0 + (n * H + h) * KV, sizeof(double) * (size_t)KV);
        else memset(S, 0, sizeof(double) * (size_t)KV);
        for (int64_t t = 0; t < L; ++t) {
            const float *kt = k + ((t0 + t) * H + h) * K;
            const float *gt = g + ((t0 + t) * H + h) * K;
            const float *vt = v + ((t0 + t) * H + h) * V;
            const double *prev = S + t * KV;
            double *cur = S + (t + 1) * KV;
            for (int64_t i = 0; i < K; ++i) {
                const double decay = exp((double)gt[i]);
                for (int64_t j = 0; j < V; ++j)
                    cur[i * V + j] = decay * prev[i * V + j] + (double)kt[i] * (double)vt[j];
            }
        }
        /* reverse sweep: U holds dL/dS_t once the term of o_t is added */
        if (dht) memcpy(U, dht + (n * H + h) * KV, sizeof(double) * (size_t)KV);
        else memset(U, 0, sizeof(double) * (size_t)KV);
        for (int64_t t = L - 1; t >= 0; --t) {
            const int64_t row = (t0 + t) * H + h;
            const float *qt = q + row * K, *kt = k + row * K, *gt = g + row * K;
            const float *vt = v + row * V, *dot = do_ + row * V;
            const double *St = S + (t + 1) * KV, *Sp = S + t * KV;
            for (int64_t i = 0; i < K; ++i)
                for (int64_t j = 0; j < V; ++j) U[i * V + j] += scale * (double)qt[i] * (double)dot[j];
            for (int64_t i = 0; i < K; ++i) {
                double aq = 0.0, ak = 0.0, ag = 0.0;
                for (int64_t j = 0; j < V; ++j) {
                    aq += St[i * V + j] * (double)dot[j];
                    ak += U[i * V + j] * (double)vt[j];
                    ag += U[i * V + j] * Sp[i * V + j];
                }
                dq[row * K + i] = scale * aq;
                dk[row * K + i] = ak;
                dg[row * K + i] = exp((double)gt[i]) * ag;
            }
            for (int64_t j = 0; j < V; ++j) {
                double a = 0.0;
                for (int64_t i = 0; i < K; ++i) a += U[i * V + j] * (double)kt[i];
                dv[row * V + j] = a;
            }
            /* dL/dS_{t-1} from S_t = diag(exp(g_t)) S_{t-1} + ... */
            for (int64_t i = 0; i < K; ++i) {
                const double decay = exp((double)gt[i]);
                for (int64_t j = 0; j < V; ++j) U[i * V + j] *= decay;
            }
        }
        if (dh0) memcpy(dh0 + (n * H + h) * KV, U, sizeof(double) * (size_t)KV);
        free(S);
        free(U);
    }
    return failed ? -1 : 0;
}

/* Threads an OpenMP parallel region of this library actually gets. */
int gla_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
