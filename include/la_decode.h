/*
 * la_decode.h -- C ABI of the MI355X (gfx950) pool-indexed recurrent-state
 * decode library for linear attention: Lightning, gated delta rule (GDN) and
 * Kimi delta attention (KDA).
 *
 * What a call computes. For every request b and value head hv:
 *   1. r = read_idx[b], w = write_idx ? write_idx[b] : r.
 *      r < 0 marks a padded request: its outputs are set to 0 and neither
 *      the pool nor the intermediate cache is read or written.
 *   2. S = pool[r, hv] (a V x K tile, k contiguous, fp32 or bf16 in the
 *      pool, fp32 in the computation).
 *   3. For t = 0..T-1 (tokens in order), with q/k head h = hv / (HV / H):
 *        Lightning:  S <- lambda[hv] * S + v_t k_t^T
 *        GDN:        S <- exp(g[b,t,hv]) * S
 *                    S <- S + beta_t (v_t - S k_t) k_t^T
 *        KDA:        S <- S diag(exp(g[b,t,hv,:]))
 *                    S <- S + beta_t (v_t - S k_t) k_t^T
 *        out[b,t,hv,:] = S q_t   (with the updated S)
 *        inter[b,t,hv] = S       (when an intermediate cache is given)
 *   4. If w >= 0: pool[w, hv] = S, in place.
 *   With a per-token slot table (see la_decode_args), the seed slot is the
 *   last accepted token's entry and step 4 becomes a write after every
 *   token to that token's entry. With cu_seqlens (a variable-length batch)
 *   request b runs its own T_b tokens of token-packed inputs.
 *
 * Sources (page titles and sections):
 *  - "fix: wire h0_indices into Lightning Attention decode for state-pool
 *    indexing" (cuLA PR #75), Description: the state is read and written
 *    through the per-request slot index (row h0_indices[i] * HV + hv of the
 *    pool), and the grid covers the active requests, not the pool rows.
 *  - FlashInfer "fp32 sibling of #3268" (gated_delta_rule_mtp), Description
 *    items 1-2, "Before vs after", "API change -- one new argument": 4D pool
 *    [pool_size, HV, V, K] read and written in place through its strides
 *    (never a silent copy); an optional separate write-slot array that
 *    defaults to the read slots, negative entries skipping the writeback;
 *    multi-token (MTP) verify with optional per-token state caching.
 *  - FlashInfer packed-QKV fix, Description: q/k/v may be head-dim slices of
 *    one fused buffer (non-compact strides), with results identical to
 *    contiguous inputs.
 *  - "[Triton/Gluon] Fused Gluon KDA decode path (950/1250)" (ROCm/aiter PR
 *    #4584), advisory review: the per-token update and output above, with
 *    q/k l2norm, the beta sigmoid and the gate fused into the kernel; and the
 *    reviewer's lesson that ambiguous or inconsistent arguments must be
 *    rejected, not silently reinterpreted.
 *
 * Conventions for every entry point:
 *  - All data pointers are DEVICE pointers; the caller owns every buffer.
 *    The library never allocates, copies, reshapes or synchronises, and
 *    keeps no state between calls.
 *  - Strides are in elements (not bytes), must be >= 0, and the innermost
 *    dimension of every tensor has stride 1.
 *  - The call is asynchronous on `stream` (a hipStream_t, NULL = the null
 *    stream). Argument checks run on the host before anything is launched:
 *    on any error status nothing is launched and no byte is touched.
 *  - B == 0 is a no-op returning LA_OK.
 *  - Device preconditions, not checked on the hot path (la_check_indices
 *    checks them): read and write slots are < pool_size; the non-negative
 *    write slots are distinct; no request's write slot equals another
 *    request's read slot (all reads are meant to see the pool as it was
 *    before the call). Breaking them is undefined behaviour.
 *  - Calls on different streams may run concurrently when their write slots
 *    are disjoint from each other's read and write slots.
 */
#ifndef LA_DECODE_H
#define LA_DECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum la_status {
    LA_OK = 0,
    LA_ERR_NULL = 1,        /* a required pointer is NULL                    */
    LA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent        */
    LA_ERR_STRIDE = 3,      /* negative stride, innermost stride != 1,
                               overlapping pool tiles or outputs, or a tile
                               whose rows span 2 GiB or more                 */
    LA_ERR_ALIGN = 4,       /* pool / cache row not 16-byte aligned, or an
                               activation not aligned to its element size    */
    LA_ERR_DTYPE = 5,       /* unknown dtype code                            */
    LA_ERR_ARG = 6,         /* argument inconsistent with the entry point
                               (e.g. beta or flags given to la_decode, an
                               unknown flag bit, gate inputs without the
                               gate flag, a nonzero reserved field)         */
    LA_ERR_UNSUPPORTED = 7, /* K or V not in {64, 128}                        */
    LA_ERR_LAUNCH = 8       /* the HIP runtime refused the launch            */
} la_status;

typedef enum la_dtype {
    LA_F32 = 0,
    LA_BF16 = 1
} la_dtype;

/* flags (GDN and KDA only; la_decode requires flags == 0) */
#define LA_F_L2NORM_QK 0x1u  /* q, k <- x / sqrt(sum x^2 + 1e-6) per head */
#define LA_F_BETA_LOGIT 0x2u /* beta holds logits; beta <- 1/(1+exp(-x))  */
#define LA_F_GATE 0x4u       /* g holds the raw gate of the gate chain    */
#define LA_F_GATE_LOWER_BOUND 0x8u /* bounded form of the gate chain     */

/* Element strides of an activation tensor [B, T, heads, (inner)]. */
typedef struct la_act_strides {
    int64_t b, t, h;
} la_act_strides;

/* Element strides of the state pool [pool_size, HV, V, K]; K stride is 1. */
typedef struct la_pool_strides {
    int64_t slot, head, row;
} la_pool_strides;

typedef struct la_decode_args {
    int32_t B;         /* requests in the batch, >= 0                       */
    int32_t T;         /* tokens per request, >= 1                          */
    int32_t H;         /* q/k heads, >= 1                                   */
    int32_t HV;        /* value heads = state tiles per slot; HV % H == 0   */
    int32_t K;         /* key width: 64 or 128                              */
    int32_t V;         /* value width: 64 or 128                            */
    int32_t pool_size; /* slots in the pool, >= 1                           */
    uint32_t flags;    /* LA_F_* bits                                       */
    la_dtype qkv_dtype; /* dtype of q, k, v                                 */
    la_dtype out_dtype; /* dtype of out                                     */
    la_dtype state_dtype; /* dtype of pool and inter: LA_F32, or LA_BF16
                             (widened exactly to fp32 on load; all math in
                             fp32; rounded to nearest even on store)        */

    const void *q;     /* [B, T, H, K]   */
    la_act_strides sq;
    const void *k;     /* [B, T, H, K]   */
    la_act_strides sk;
    const void *v;     /* [B, T, HV, V]  */
    la_act_strides sv;
    /* Decay input, fp32:
     *   la_decode:      lambda[HV] decay factors (contiguous), or NULL for
     *                   lambda[hv] = exp(-2^(-8 (hv+1) / HV)); sg unused
     *   gdn_decode_mtp: g[B, T, HV] log-decay (sg.b, sg.t, sg.h)
     *   kda_decode_mtp: g[B, T, HV, K] log-decay, K stride 1               */
    const float *g;
    la_act_strides sg;
    /* beta[B, T, HV] fp32 (GDN, KDA; logits when LA_F_BETA_LOGIT);
     * must be NULL for la_decode */
    const float *beta;
    la_act_strides sbeta;

    void *pool;        /* [pool_size, HV, V, K] in state_dtype, updated in
                          place; base and every row start 16-byte aligned  */
    la_pool_strides sp;
    const int32_t *read_idx;  /* [B] contiguous                             */
    const int32_t *write_idx; /* [B] contiguous, or NULL (= read_idx)       */
    void *inter;       /* [B, T, HV, V, K] contiguous, state_dtype, or NULL */
    void *out;         /* [B, T, HV, V] in out_dtype                        */
    la_act_strides so;

    /* Paged per-token state slots for speculative decoding (aiter KDA page,
     * advisory review), or NULL. token_slots is a [B, T] int32 table with
     * row stride token_slots_stride (>= T, in elements; a flat table is
     * rejected rather than guessed at). Request b reads its seed state from
     * slot token_slots[b][num_accepted[b] - 1], the slot of its last
     * accepted token, and after each token t writes the state to slot
     * token_slots[b][t] (a negative entry skips that write). When the table
     * is given, read_idx and write_idx must be NULL and num_accepted ([B],
     * contiguous) is required. A request whose num_accepted is outside
     * [1, T] or whose seed entry is negative is padding: zero outputs, no
     * pool or cache access. */
    const int32_t *token_slots;
    int64_t token_slots_stride;
    const int32_t *num_accepted;

    /* Per-token update records (aiter KDA page, advisory review: each
     * token's update kept as an (a, k, err) triple instead of a full
     * per-token state), or NULL:
     * [B, T, HV, 2K + V] fp32, contiguous, 16-byte aligned. Record t of
     * (b, hv) holds a_t[K] (the decay: the KDA factors exp(g), or the GDN /
     * Lightning scalar repeated K times), k_t[K] (the key as used, after
     * l2norm) and err_t[V] (the rank-1 coefficient: beta (v - S k) for
     * GDN/KDA, v for Lightning), so that S_t = S_{t-1} diag(a_t) +
     * err_t k_t^T exactly as the kernel computed it. la_replay rebuilds S_t
     * from the seed state; 2K + V floats per token instead of V K. Written
     * for active requests only. */
    float *factors;

    /* Variable-length batch (aiter KDA page, summary: the decode kernel takes
     * varlen batches; the token-packed layout below is this library's
     * reading), or NULL: cu_seqlens[B + 1] int32 offsets, contiguous.
     * Request b owns tokens cu_seqlens[b] .. cu_seqlens[b+1] - 1 of
     * token-packed per-token arrays and runs T_b = cu_seqlens[b+1] -
     * cu_seqlens[b] tokens; T is an upper bound on every T_b. q, k, v, g,
     * beta and out are then indexed by the flat token number through their
     * t strides (their b strides are ignored); inter is
     * [total_tokens, HV, V, K] and factors [total_tokens, HV, 2K + V], both
     * contiguous. A request with T_b = 0 copies its read state to its write
     * slot. With total_tokens = 0 the per-token arrays are empty and q, k,
     * v, g, beta and out may be NULL (no request can index them). With a
     * slot table, num_accepted must lie in [1, T_b] (otherwise
     * the request is padding). Device precondition (la_check_cu_seqlens
     * checks it): 0 <= cu_seqlens[b] <= cu_seqlens[b+1] <= total_tokens and
     * T_b <= T. A request that breaks it is skipped entirely: no output is
     * written and neither the pool nor the cache is accessed. */
    const int32_t *cu_seqlens;
    int32_t total_tokens; /* rows of the token-packed arrays (cu_seqlens
                             given), >= 0; ignored otherwise              */
    int32_t reserved;     /* must be 0                                    */

    /* In-kernel gate chain (aiter KDA page, advisory review: the wrapper
     * takes A_log, dt_bias with HV*K entries, lower_bound and
     * use_gate_in_kernel, and gate inputs given without the switch must be
     * refused; the pages do not state the formula, this is the library's
     * reading). With LA_F_GATE (GDN, KDA), g holds the raw gate x and the
     * log-decay becomes
     *     -exp(A_log[hv]) * softplus(x + dt_bias)
     * or, with LA_F_GATE_LOWER_BOUND,
     *     lower_bound * sigmoid(exp(A_log[hv]) * (x + dt_bias)),
     * where dt_bias is dt_bias[hv] (GDN) or dt_bias[hv][k] (KDA); the decay
     * is exp of it, as without the chain. A_log [HV] and dt_bias ([HV] or
     * [HV, K]) are fp32, contiguous, and required with LA_F_GATE (else
     * LA_ERR_NULL); either given without LA_F_GATE, or
     * LA_F_GATE_LOWER_BOUND without LA_F_GATE, is LA_ERR_ARG. */
    const float *A_log;
    const float *dt_bias;
    float lower_bound;    /* with LA_F_GATE_LOWER_BOUND: finite, < 0      */
    int32_t reserved2;    /* must be 0                                    */
} la_decode_args;

/* Arguments of la_replay. */
typedef struct la_replay_args {
    int32_t B;          /* requests, >= 0                                    */
    int32_t T;          /* records per request in `factors`, >= 1            */
    int32_t HV;         /* value heads, >= 1                                 */
    int32_t K;          /* 64 or 128                                         */
    int32_t V;          /* 64 or 128                                         */
    int32_t pool_size;  /* >= 1                                              */
    la_dtype state_dtype;
    const float *factors;       /* [B, T, HV, 2K + V] fp32, contiguous      */
    void *pool;                 /* [pool_size, HV, V, K], as in la_decode   */
    la_pool_strides sp;
    const int32_t *read_idx;    /* [B] seed slots; negative: skip request   */
    const int32_t *write_idx;   /* [B] or NULL (= read_idx); negative: skip */
    const int32_t *num_tokens;  /* [B] records to apply; a value outside
                                   [0, T] (with cu_seqlens: [0, T_b]) skips
                                   the request                              */
    const int32_t *cu_seqlens;  /* NULL, or [B + 1] offsets as in
                                   la_decode_args: factors is then
                                   [total_tokens, HV, 2K + V] (may be NULL
                                   when total_tokens = 0)                   */
    int32_t total_tokens;       /* with cu_seqlens, >= 0                    */
    int32_t reserved;           /* must be 0                                */
} la_replay_args;

/* Lightning decode (cuLA page): S <- lambda_h S + v k^T, o = S q.
 * Requires beta == NULL and flags == 0. */
la_status la_decode(const la_decode_args *args, void *stream);

/* Gated delta rule decode, single- or multi-token (FlashInfer
 * gated_delta_rule_mtp page): scalar decay exp(g) then the delta update. */
la_status gdn_decode_mtp(const la_decode_args *args, void *stream);

/* KDA decode (aiter KDA page): per-key-channel decay exp(g[:]) then the
 * delta update. */
la_status kda_decode_mtp(const la_decode_args *args, void *stream);

/* Rebuild states from per-token update records (aiter KDA page: cached
 * (a,k,err) updates, the state pool written only for the accepted tokens).
 * For every request b and value head hv: S = pool[read_idx[b], hv]; for
 * t < num_tokens[b]: S <- S diag(a_t) + err_t k_t^T (the records that
 * la_decode, gdn_decode_mtp or kda_decode_mtp wrote); then
 * pool[write_idx[b], hv] = S when the write slot is not negative. Same
 * device preconditions on the slots as the decode calls; on fp32 pools the
 * result equals the per-token cache of the decode call bit for bit. */
la_status la_replay(const la_replay_args *args, void *stream);

/* Debug validator of the device preconditions above (the aiter review's
 * failure modes: slots out of range, snapshots written into other
 * sequences' slots). Writes a bit set to *dev_result (device int32):
 *   1 = a read slot >= pool_size,  2 = a write slot >= pool_size,
 *   4 = two requests write the same slot,
 *   8 = a request writes a slot another request reads.
 * 0 means the index set is valid. write_idx may be NULL (= read_idx).
 * Asynchronous on `stream`: a one-thread kernel clears *dev_result, then
 * one workgroup per request compares it with every other request and ORs
 * its findings in. B == 0 writes 0. */
la_status la_check_indices(int32_t B, int32_t pool_size,
                           const int32_t *read_idx, const int32_t *write_idx,
                           int32_t *dev_result, void *stream);

/* Debug validator for the paged per-token slot table (same conventions as
 * la_check_indices). Bits written to *dev_result:
 *   1 = a seed slot >= pool_size,  2 = a table entry >= pool_size,
 *   4 = two requests write the same slot,
 *   8 = a request writes another request's seed slot,
 *   16 = a num_accepted entry outside [1, T] (that request is padding).
 * table_stride must be >= T. */
la_status la_check_token_slots(int32_t B, int32_t T, int32_t pool_size,
                               const int32_t *token_slots,
                               int64_t table_stride,
                               const int32_t *num_accepted,
                               int32_t *dev_result, void *stream);

/* Debug validator of the variable-length offsets (same conventions as
 * la_check_indices). Bits written to *dev_result:
 *   1 = an offset outside [0, total_tokens],
 *   2 = a request with a negative token count or more than T tokens.
 * Requests flagged here are skipped by the decode and replay calls. */
la_status la_check_cu_seqlens(int32_t B, int32_t T, int32_t total_tokens,
                              const int32_t *cu_seqlens, int32_t *dev_result,
                              void *stream);

/* Variant codes of la_decode_kernel_info: the decode entry point a query
 * stands for. */
typedef enum la_variant {
    LA_VARIANT_LIGHTNING = 0, /* la_decode      */
    LA_VARIANT_GDN = 1,       /* gdn_decode_mtp */
    LA_VARIANT_KDA = 2        /* kda_decode_mtp */
} la_variant;

/* The kernel a decode call selects, its launch shape and its register
 * budget on the current device. */
typedef struct la_kernel_info {
    const char *kernel;     /* "decode_kernel" (any call),
                               "decode1_kernel" (one token, large grids),
                               "decode_packed_kernel" (one token, bf16 pool)
                               or "none" (B = 0: nothing is launched);
                               static storage owned by the library */
    int32_t grid_blocks;    /* workgroups: B * HV (four per tile in
                               decode1_kernel at K = V = 128)              */
    int32_t block_threads;  /* threads per workgroup                       */
    int32_t lds_bytes;      /* dynamic LDS per workgroup: the token records
                               of one round, plus a per-wave staging area
                               in the instances that pass the final state
                               through LDS before storing it               */
    int32_t vgprs;          /* architected VGPRs per lane                  */
    int32_t scratch_bytes;  /* private (spill) memory per lane             */
    int32_t blocks_per_cu;  /* workgroups resident on one compute unit     */
    int32_t waves_per_simd; /* blocks_per_cu * waves per workgroup / 4     */
    int32_t tokens_per_round; /* token records staged in LDS per round (the
                               instance's; lds_bytes holds min(T, this) of
                               them); 0 for decode1_kernel, which stages
                               nothing, 1 for decode_packed_kernel         */
} la_kernel_info;

/* Describe the kernel that the decode call `args` of `variant` would run
 * (not an operation of the method: a report of this library's dispatch, for
 * callers that size batches or check occupancy). Host only: launches
 * nothing and reads no device memory. Runs the entry point's host checks
 * first and returns the status the call itself would return, leaving *info
 * untouched on error. LA_ERR_NULL for a NULL info, LA_ERR_ARG for an unknown
 * variant, LA_ERR_LAUNCH when the HIP runtime cannot report the kernel's
 * attributes (for instance without a device). */
la_status la_decode_kernel_info(int32_t variant, const la_decode_args *args,
                                la_kernel_info *info);

/* Static description of a status code; never NULL. */
const char *la_status_string(la_status status);

/* Library version as major * 100 + minor (2.00: state_dtype and paged
 * per-token slots in la_decode_args; 2.10: variable-length batches; 2.20:
 * the in-kernel gate chain; 2.30: la_decode_kernel_info). */
int32_t la_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LA_DECODE_H */
