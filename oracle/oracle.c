/*
 * oracle.c -- plain fp64 CPU reference for pool-indexed recurrent-state decode
 * of linear attention: Lightning, gated delta rule (GDN) and Kimi delta
 * attention (KDA).
 *
 * TEST INFRASTRUCTURE. This file is the parity oracle. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load or call it.
 * It shares no code, header, table or helper with the GPU library, and the
 * GPU library never calls it.
 *
 * It evaluates the recurrence directly, one request and one value head at a
 * time, one token after another, in scalar double-precision loops with no
 * blocking, fusion or reordering. Where it follows the pages:
 *
 *  - "[Triton/Gluon] Fused Gluon KDA decode path (950/1250)" (ROCm/aiter
 *    PR #4584), advisory review, summary paragraph: per token the state is
 *    decayed by exp(g_t), then corrected by beta_t * k_t (x) (v_t - S^T k_t),
 *    and the token's output is S^T q_t with the updated state; q/k l2norm and
 *    the beta sigmoid are fused into that kernel's prologue.
 *  - "fix: wire h0_indices into Lightning Attention decode for state-pool
 *    indexing" (cuLA PR #75), Description / What changed: request i reads and
 *    writes pool row h0_indices[i] * HV + hv, not the batch position.
 *  - FlashInfer "fp32 sibling of #3268" description (4D pool
 *    [pool_size, HV, V, K]; "Separate read/write slots"; "API change -- one
 *    new argument"): the write slot defaults to the read slot and a negative
 *    write slot skips the writeback; a negative read slot is padding (the
 *    write side mirrors the read side's -1 padding).
 *
 * Storage orientation: the pool stores each state tile as S[v][k] with k
 * contiguous (the [pool_size, HV, V, K] layout). The pages write the update
 * with the mathematical state as K x V (S^T k); in storage that read-out is
 * the row-wise dot product u[v] = sum_k S[v][k] * k[k].
 *
 * Readings where the pages are silent:
 *  - Lightning: the pages name the operation only. The update is the
 *    decay-masked linear-attention recurrence S <- lambda_h * S + v k^T,
 *    o = S q, with the standard per-head decay lambda_h = exp(-2^(-8(h+1)/H))
 *    over the value heads when no decay array is given.
 *  - g is a log-decay: GDN alpha = exp(g) (scalar per token and value head),
 *    KDA e = exp(g) (one factor per key channel).
 *  - l2norm is x / sqrt(sum x^2 + 1e-6).
 *  - Value head hv uses q/k head h = hv / (HV / H).
 *  - A padded request (negative read slot) writes zeros to its outputs and
 *    touches neither the pool nor the intermediate cache.
 *  - The intermediate cache entry [b, t, hv] is the state after token t,
 *    written for every active request whatever its write slot.
 *  - All reads see the pool as it was before the call (pool_in); all writes
 *    go to pool_out.
 *
 * Paged per-token slots (aiter KDA page, advisory review: paged per-token
 * state slots for speculative decoding, the seed slot being the table entry
 * of the last accepted token, and the reviewer's demand that the table be
 * two-dimensional and the accepted count at least one): with a slot table
 * given, request b reads its state from slot table[b][num_accepted[b] - 1]
 * and, after each token t, writes the state to slot table[b][t] when that
 * entry is not negative. A request whose accepted count is outside [1, T]
 * or whose seed entry is negative is padding, as above.
 *
 * Factor records (aiter KDA page, advisory review: each token's update kept
 * as an (a, k, err) triple rather than as a full state; its benchmark note: not writing every per-token state saves
 * runtime as tokens and batch grow): instead of the state after token t, a
 * record [a | k | err] of 2K + V values lets the state be rebuilt as
 * S_t = S_{t-1} diag(a_t) + err_t k_t^T. Here a_t is the token's decay (the
 * KDA factors, or the GDN/Lightning scalar repeated K times), k_t the key as
 * used (after l2norm) and err_t the rank-1 coefficient: beta (v - S k) for
 * the delta rules, v for Lightning. oracle_replay applies n such records.
 *
 * Variable-length batches (aiter KDA page, summary: the decode kernel takes
 * varlen batches; the pages give no layout): with cumulative offsets
 * cu_seqlens[B + 1], request b owns tokens cu_seqlens[b] .. cu_seqlens[b+1]-1
 * of token-packed activations, i.e. T_b = cu_seqlens[b+1] - cu_seqlens[b]
 * tokens, and every per-token array (q, k, v, g, beta, out, inter, factors) is
 * indexed by that flat token number instead of (b, t). T is then an upper
 * bound on T_b. A request with T_b = 0 runs no token: its state is written to
 * its write slot unchanged. With a slot table, the accepted count must lie in
 * [1, T_b].
 *
 * In-kernel gate chain (aiter KDA page, advisory review: the wrapper takes
 * A_log, dt_bias with HV*K entries and lower_bound, and gate inputs given
 * without use_gate_in_kernel must be refused). The pages name the inputs
 * but not the formula; this oracle takes the plainest reading, the gated
 * log-decay of the delta-rule models, and marks it "parity unpinned" against
 * the pages. With the gate flag, g holds the raw gate x and the log-decay is
 *     g' = -exp(A_log[hv]) * softplus(x + dt_bias)              (default)
 *     g' = lower_bound * sigmoid(exp(A_log[hv]) * (x + dt_bias)) (bounded)
 * with dt_bias[hv] (GDN, one per value head) or dt_bias[hv][k] (KDA, one per
 * key channel); the decay is exp(g') as before.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_LIGHTNING 0
#define ORACLE_GDN 1
#define ORACLE_KDA 2

#define ORACLE_L2NORM_QK 1
#define ORACLE_BETA_LOGIT 2
#define ORACLE_GATE 4             /* g is the raw gate of the gate chain */
#define ORACLE_GATE_LOWER_BOUND 8 /* bounded (sigmoid) form of the chain */

#define ORACLE_L2NORM_EPS 1e-6

/* x <- x / sqrt(sum x^2 + eps): the in-kernel l2norm of the KDA page. */
static void l2_normalise(double *x, int n)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i)
        ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss + ORACLE_L2NORM_EPS);
    for (int i = 0; i < n; ++i)
        x[i] *= inv;
}

/* The gate chain's log-decay for raw gate x (see the header comment). */
static double gate_chain(double x, double a_log, double dt, int bounded,
                         double lower_bound)
{
    const double z = x + dt;
    if (bounded)
        return lower_bound / (1.0 + exp(-exp(a_log) * z));
    return -exp(a_log) * log1p(exp(z));
}

/* The standard Lightning Attention per-head decay. */
static double lightning_decay(int head, int num_heads)
{
    return exp(-pow(2.0, -8.0 * (double)(head + 1) / (double)num_heads));
}

/*
 * Returns 0 on success, -1 on a bad argument, -2 if memory ran out.
 *
 * Layouts (all contiguous, row-major):
 *   q, k      [B][T][H][K]
 *   v         [B][T][HV][V]
 *   g         Lightning: [HV] decay factors, or NULL for lightning_decay();
 *             GDN: [B][T][HV] log-decay; KDA: [B][T][HV][K] log-decay
 *   beta      [B][T][HV] (GDN, KDA); ignored for Lightning
 *   pool_in   [pool_size][HV][V][K]  the pool before the call (read only)
 *   pool_out  [pool_size][HV][V][K]  holds a copy of pool_in on entry;
 *                                    write slots are overwritten
 *   read_idx, write_idx  [B]; write_idx may be NULL (= read_idx)
 *   out       [B][T][HV][V]
 *   inter     [B][T][HV][V][K] or NULL
 *   slots     [B][slots_stride] per-token slot table, or NULL; when given,
 *             read_idx and write_idx are ignored and accepted[B] is used
 *   factors   [B][T][HV][2K + V] per-token records, or NULL
 *   cu_seqlens  NULL, or [B + 1] non-decreasing offsets in [0, total] with
 *             cu_seqlens[b+1] - cu_seqlens[b] <= T; then every [B][T] pair
 *             of dimensions above is one [total] token dimension
 *   A_log     [HV], dt_bias [HV] (GDN) or [HV][K] (KDA), lower_bound: the
 *             gate chain, used when flags has ORACLE_GATE
 */
int oracle_decode(int variant, int B, int T, int H, int HV, int K, int V,
                  int flags, const double *q, const double *k, const double *v,
                  const double *g, const double *beta, int pool_size,
                  const double *pool_in, double *pool_out,
                  const int32_t *read_idx, const int32_t *write_idx,
                  double *out, double *inter, const int32_t *slots,
                  int slots_stride, const int32_t *accepted, double *factors,
                  const int32_t *cu_seqlens, int total, const double *A_log,
                  const double *dt_bias, double lower_bound)
{
    if (B < 0 || T < 1 || H < 1 || HV < 1 || K < 1 || V < 1 || HV % H != 0)
        return -1;
    const int gate = (flags & ORACLE_GATE) != 0;
    const int bounded = (flags & ORACLE_GATE_LOWER_BOUND) != 0;
    if (gate && (variant == ORACLE_LIGHTNING || !A_log || !dt_bias))
        return -1;
    if (bounded && !gate)
        return -1;
    if (cu_seqlens)
        for (int b = 0; b < B; ++b)
            if (cu_seqlens[b] < 0 || cu_seqlens[b + 1] < cu_seqlens[b] ||
                cu_seqlens[b + 1] > total ||
                cu_seqlens[b + 1] - cu_seqlens[b] > T)
                return -1;
    if (variant != ORACLE_LIGHTNING && variant != ORACLE_GDN &&
        variant != ORACLE_KDA)
        return -1;
    if (slots && (slots_stride < T || !accepted))
        return -1;

    const size_t tile = (size_t)V * (size_t)K;
    double *S = (double *)malloc(tile * sizeof(double));
    double *qv = (double *)malloc((size_t)K * sizeof(double));
    double *kv = (double *)malloc((size_t)K * sizeof(double));
    double *kdec = (double *)malloc((size_t)K * sizeof(double));
    if (!S || !qv || !kv || !kdec) {
        free(S);
        free(qv);
        free(kv);
        free(kdec);
        return -2;
    }
    const int group = HV / H;

    for (int b = 0; b < B; ++b) {
        /* tokens of request b and the flat number of its first token */
        const int Tb = cu_seqlens ? cu_seqlens[b + 1] - cu_seqlens[b] : T;
        const size_t tok0 = cu_seqlens ? (size_t)cu_seqlens[b] : (size_t)b * T;
        int r, w;
        if (slots) {
            const int na = accepted[b];
            r = (na >= 1 && na <= Tb)
                    ? slots[(size_t)b * slots_stride + na - 1]
                    : -1;
            w = -1; /* per-token writes instead of one final write */
            for (int t = 0; t < T; ++t)
                if (slots[(size_t)b * slots_stride + t] >= pool_size) {
                    free(S);
                    free(qv);
                    free(kv);
                    free(kdec);
                    return -1;
                }
        } else {
            r = read_idx[b];
            w = write_idx ? write_idx[b] : r;
        }
        if (r >= pool_size || w >= pool_size) {
            free(S);
            free(qv);
            free(kv);
            free(kdec);
            return -1;
        }
        for (int hv = 0; hv < HV; ++hv) {
            if (r < 0) {
                /* padded request: zero outputs, nothing else */
                for (int t = 0; t < Tb; ++t)
                    for (int i = 0; i < V; ++i)
                        out[((tok0 + t) * HV + hv) * V + i] = 0.0;
                continue;
            }
            const int h = hv / group;
            memcpy(S, pool_in + ((size_t)r * HV + hv) * tile,
                   tile * sizeof(double));

            for (int t = 0; t < Tb; ++t) {
                const size_t qk_off = ((tok0 + t) * H + h) * K;
                const size_t v_off = ((tok0 + t) * HV + hv) * V;
                const size_t bt = (tok0 + t) * HV + hv;
                memcpy(qv, q + qk_off, (size_t)K * sizeof(double));
                memcpy(kv, k + qk_off, (size_t)K * sizeof(double));
                if (flags & ORACLE_L2NORM_QK) {
                    l2_normalise(qv, K);
                    l2_normalise(kv, K);
                }
                const double *vv = v + v_off;

                double *rec =
                    factors ? factors + bt * (size_t)(2 * K + V) : NULL;
                if (rec)
                    memcpy(rec + K, kv, (size_t)K * sizeof(double));
                if (variant == ORACLE_LIGHTNING) {
                    const double lam = g ? g[hv] : lightning_decay(hv, HV);
                    if (rec) {
                        for (int j = 0; j < K; ++j)
                            rec[j] = lam;
                        for (int i = 0; i < V; ++i)
                            rec[2 * K + i] = vv[i];
                    }
                    /* S <- lambda * S + v k^T */
                    for (int i = 0; i < V; ++i)
                        for (int j = 0; j < K; ++j)
                            S[(size_t)i * K + j] =
                                lam * S[(size_t)i * K + j] + vv[i] * kv[j];
                } else {
                    double bb = beta[bt];
                    if (flags & ORACLE_BETA_LOGIT)
                        bb = 1.0 / (1.0 + exp(-bb));
                    /* decay: S <- alpha S (GDN) or S <- S diag(exp g) (KDA) */
                    if (variant == ORACLE_GDN) {
                        const double alpha =
                            exp(gate ? gate_chain(g[bt], A_log[hv], dt_bias[hv],
                                                  bounded, lower_bound)
                                     : g[bt]);
                        for (size_t e = 0; e < tile; ++e)
                            S[e] *= alpha;
                        if (rec)
                            for (int j = 0; j < K; ++j)
                                rec[j] = alpha;
                    } else {
                        const double *gk = g + bt * (size_t)K;
                        /* the channel decays of this token */
                        double *ek = kdec;
                        for (int j = 0; j < K; ++j)
                            ek[j] = exp(gate ? gate_chain(gk[j], A_log[hv],
                                                          dt_bias[(size_t)hv * K + j],
                                                          bounded, lower_bound)
                                             : gk[j]);
                        for (int i = 0; i < V; ++i)
                            for (int j = 0; j < K; ++j)
                                S[(size_t)i * K + j] *= ek[j];
                        if (rec)
                            for (int j = 0; j < K; ++j)
                                rec[j] = ek[j];
                    }
                    /* delta rule: S <- S + beta (v - S k) k^T, one row at a
                     * time (row i's read-out uses only row i) */
                    for (int i = 0; i < V; ++i) {
                        double u = 0.0;
                        for (int j = 0; j < K; ++j)
                            u += S[(size_t)i * K + j] * kv[j];
                        const double c = bb * (vv[i] - u);
                        for (int j = 0; j < K; ++j)
                            S[(size_t)i * K + j] += c * kv[j];
                        if (rec)
                            rec[2 * K + i] = c;
                    }
                }
                /* o = S q with the updated state */
                for (int i = 0; i < V; ++i) {
                    double o = 0.0;
                    for (int j = 0; j < K; ++j)
                        o += S[(size_t)i * K + j] * qv[j];
                    out[v_off + i] = o;
                }
                if (inter)
                    memcpy(inter + bt * tile, S, tile * sizeof(double));
                if (slots) {
                    const int ws = slots[(size_t)b * slots_stride + t];
                    if (ws >= 0)
                        memcpy(pool_out + ((size_t)ws * HV + hv) * tile, S,
                               tile * sizeof(double));
                }
            }
            if (w >= 0)
                memcpy(pool_out + ((size_t)w * HV + hv) * tile, S,
                       tile * sizeof(double));
        }
    }
    free(S);
    free(qv);
    free(kv);
    free(kdec);
    return 0;
}

/*
 * Rebuild states from factor records: for each request b with
 * 0 <= ntok[b] <= T and read slot r = read_idx[b] >= 0, start from
 * pool_in[r, hv] and apply records t = 0 .. ntok[b] - 1 of that request,
 * S <- S diag(a_t) + err_t k_t^T; then write S to pool_out[w, hv] with
 * w = write_idx ? write_idx[b] : r when w >= 0. Requests with a negative
 * read slot or ntok outside [0, T] are skipped.
 * factors: [B][T][HV][2K + V]; with cu_seqlens (as in oracle_decode),
 * [total][HV][2K + V] by flat token number, and ntok[b] must lie in
 * [0, T_b]. Returns 0, or -1 on a bad argument.
 */
int oracle_replay(int B, int T, int HV, int K, int V, const double *factors,
                  int pool_size, const double *pool_in, double *pool_out,
                  const int32_t *read_idx, const int32_t *write_idx,
                  const int32_t *ntok, const int32_t *cu_seqlens, int total)
{
    if (B < 0 || T < 1 || HV < 1 || K < 1 || V < 1)
        return -1;
    if (cu_seqlens)
        for (int b = 0; b < B; ++b)
            if (cu_seqlens[b] < 0 || cu_seqlens[b + 1] < cu_seqlens[b] ||
                cu_seqlens[b + 1] > total ||
                cu_seqlens[b + 1] - cu_seqlens[b] > T)
                return -1;
    const size_t tile = (size_t)V * (size_t)K;
    const size_t rsz = (size_t)(2 * K + V);
    double *S = (double *)malloc(tile * sizeof(double));
    if (!S)
        return -2;
    for (int b = 0; b < B; ++b) {
        const int r = read_idx[b];
        const int w = write_idx ? write_idx[b] : r;
        const int n = ntok[b];
        const int Tb = cu_seqlens ? cu_seqlens[b + 1] - cu_seqlens[b] : T;
        const size_t tok0 = cu_seqlens ? (size_t)cu_seqlens[b] : (size_t)b * T;
        if (r >= pool_size || w >= pool_size) {
            free(S);
            return -1;
        }
        if (r < 0 || n < 0 || n > Tb)
            continue;
        for (int hv = 0; hv < HV; ++hv) {
            memcpy(S, pool_in + ((size_t)r * HV + hv) * tile,
                   tile * sizeof(double));
            for (int t = 0; t < n; ++t) {
                const double *rec = factors + ((tok0 + t) * HV + hv) * rsz;
                const double *a = rec, *kk = rec + K, *err = rec + 2 * K;
                for (int i = 0; i < V; ++i)
                    for (int j = 0; j < K; ++j)
                        S[(size_t)i * K + j] =
                            S[(size_t)i * K + j] * a[j] + err[i] * kk[j];
            }
            if (w >= 0)
                memcpy(pool_out + ((size_t)w * HV + hv) * tile, S,
                       tile * sizeof(double));
        }
    }
    free(S);
    return 0;
}
