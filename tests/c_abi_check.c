/*
 * c_abi_check.c -- drives the decode library through include/la_decode.h
 * alone (no Python, no PyTorch) and compares with the fp64 oracle.
 *
 * TEST INFRASTRUCTURE: it links the oracle (oracle/liboracle.so), which only
 * tests may use. Built by __graft_entry__.build() next to this file
 * (tests/c_abi_check); run by tests/test_c_abi.py on a GPU.
 *
 * One gated-delta-rule call: B = 3 requests, T = 2 tokens, H = 2 q/k heads,
 * HV = 4 value heads, K = V = 128, fp32 inputs and state, a pool of 8 slots,
 * read slots {5, 0, 3}, write slots {1, 2, -1}, in-kernel l2norm and beta
 * sigmoid, per-token state cache. Inputs come from a fixed xorshift stream
 * and feed both sides. Exit status 0 when outputs, written slots and the
 * cache agree to 1e-4 relative (the fp32 tolerance), every other slot is
 * untouched, and the host rejects a malformed call; 1 otherwise.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "la_decode.h"

/* oracle/oracle.c (test infrastructure) */
int oracle_decode(int variant, int B, int T, int H, int HV, int K, int V,
                  int flags, const double *q, const double *k, const double *v,
                  const double *g, const double *beta, int pool_size,
                  const double *pool_in, double *pool_out,
                  const int32_t *read_idx, const int32_t *write_idx,
                  double *out, double *inter, const int32_t *slots,
                  int slots_stride, const int32_t *accepted, double *factors,
                  const int32_t *cu_seqlens, int total, const double *A_log,
                  const double *dt_bias, double lower_bound);

enum { B = 3, T = 2, H = 2, HV = 4, K = 128, V = 128, P = 8 };

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

/* xorshift64*, mapped to [-1, 1) */
static float uniform(void)
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    const uint64_t x = rng_state * 0x2545f4914f6cdd1dull;
    return (float)((double)(x >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

#define CHECK_HIP(call)                                                    \
    do {                                                                   \
        hipError_t e_ = (call);                                            \
        if (e_ != hipSuccess) {                                            \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_)); \
            return 1;                                                      \
        }                                                                  \
    } while (0)

static double rel_err(const float *got, const double *ref, size_t n)
{
    double num = 0.0, den = 1e-30;
    for (size_t i = 0; i < n; ++i) {
        const double d = fabs((double)got[i] - ref[i]);
        if (!(d <= num))
            num = d; /* also catches NaN */
        if (fabs(ref[i]) > den)
            den = fabs(ref[i]);
    }
    return num / den;
}

int main(void)
{
    const size_t nq = (size_t)B * T * H * K, nv = (size_t)B * T * HV * V;
    const size_t ng = (size_t)B * T * HV, tile = (size_t)V * K;
    const size_t npool = (size_t)P * HV * tile, nout = nv;
    const size_t ninter = (size_t)B * T * HV * tile;
    const int32_t ridx[B] = {5, 0, 3}, widx[B] = {1, 2, -1};

    float *hq = malloc(nq * 4), *hk = malloc(nq * 4), *hv = malloc(nv * 4);
    float *hg = malloc(ng * 4), *hb = malloc(ng * 4);
    float *hpool = malloc(npool * 4), *hout = malloc(nout * 4);
    float *hpool_after = malloc(npool * 4), *hinter = malloc(ninter * 4);
    double *dq = malloc(nq * 8), *dk = malloc(nq * 8), *dv = malloc(nv * 8);
    double *dg = malloc(ng * 8), *db = malloc(ng * 8);
    double *dpool = malloc(npool * 8), *dpool_out = malloc(npool * 8);
    double *dout = malloc(nout * 8), *dinter = malloc(ninter * 8);
    if (!hq || !hk || !hv || !hg || !hb || !hpool || !hout || !hpool_after ||
        !hinter || !dq || !dk || !dv || !dg || !db || !dpool || !dpool_out ||
        !dout || !dinter) {
        fprintf(stderr, "out of host memory\n");
        return 1;
    }
    for (size_t i = 0; i < nq; ++i) hq[i] = uniform();
    for (size_t i = 0; i < nq; ++i) hk[i] = uniform();
    for (size_t i = 0; i < nv; ++i) hv[i] = uniform();
    for (size_t i = 0; i < ng; ++i) hg[i] = 0.25f * (uniform() - 1.0f);
    for (size_t i = 0; i < ng; ++i) hb[i] = 2.0f * uniform();
    for (size_t i = 0; i < npool; ++i) hpool[i] = 0.1f * uniform();
    for (size_t i = 0; i < nq; ++i) { dq[i] = hq[i]; dk[i] = hk[i]; }
    for (size_t i = 0; i < nv; ++i) dv[i] = hv[i];
    for (size_t i = 0; i < ng; ++i) { dg[i] = hg[i]; db[i] = hb[i]; }
    for (size_t i = 0; i < npool; ++i) dpool[i] = dpool_out[i] = hpool[i];

    const int flags = LA_F_L2NORM_QK | LA_F_BETA_LOGIT;
    if (oracle_decode(1, B, T, H, HV, K, V, flags, dq, dk, dv, dg, db, P,
                      dpool, dpool_out, ridx, widx, dout, dinter, NULL, 0,
                      NULL, NULL, NULL, 0, NULL, NULL, 0.0) != 0) {
        fprintf(stderr, "oracle rejected the call\n");
        return 1;
    }

    void *q, *k, *v, *g, *beta, *pool, *out, *inter, *ri, *wi;
    CHECK_HIP(hipMalloc(&q, nq * 4));
    CHECK_HIP(hipMalloc(&k, nq * 4));
    CHECK_HIP(hipMalloc(&v, nv * 4));
    CHECK_HIP(hipMalloc(&g, ng * 4));
    CHECK_HIP(hipMalloc(&beta, ng * 4));
    CHECK_HIP(hipMalloc(&pool, npool * 4));
    CHECK_HIP(hipMalloc(&out, nout * 4));
    CHECK_HIP(hipMalloc(&inter, ninter * 4));
    CHECK_HIP(hipMalloc(&ri, sizeof ridx));
    CHECK_HIP(hipMalloc(&wi, sizeof widx));
    CHECK_HIP(hipMemcpy(q, hq, nq * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(k, hk, nq * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(v, hv, nv * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(g, hg, ng * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(beta, hb, ng * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(pool, hpool, npool * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(ri, ridx, sizeof ridx, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(wi, widx, sizeof widx, hipMemcpyHostToDevice));

    la_decode_args a;
    memset(&a, 0, sizeof a);
    a.B = B; a.T = T; a.H = H; a.HV = HV; a.K = K; a.V = V; a.pool_size = P;
    a.flags = (uint32_t)flags;
    a.qkv_dtype = LA_F32; a.out_dtype = LA_F32; a.state_dtype = LA_F32;
    a.q = q; a.sq = (la_act_strides){T * H * K, H * K, K};
    a.k = k; a.sk = a.sq;
    a.v = v; a.sv = (la_act_strides){T * HV * V, HV * V, V};
    a.g = (const float *)g; a.sg = (la_act_strides){T * HV, HV, 1};
    a.beta = (const float *)beta; a.sbeta = a.sg;
    a.pool = pool; a.sp = (la_pool_strides){HV * (int64_t)tile, (int64_t)tile, K};
    a.read_idx = (const int32_t *)ri; a.write_idx = (const int32_t *)wi;
    a.inter = inter;
    a.out = out; a.so = a.sv;

    /* a malformed call is refused on the host and launches nothing */
    la_decode_args bad = a;
    bad.H = 3;
    if (gdn_decode_mtp(&bad, NULL) != LA_ERR_SHAPE) {
        fprintf(stderr, "HV %% H != 0 was not rejected\n");
        return 1;
    }

    int32_t *check;
    int32_t flags_found = -1;
    CHECK_HIP(hipMalloc((void **)&check, 4));
    if (la_check_indices(B, P, (const int32_t *)ri, (const int32_t *)wi,
                         check, NULL) != LA_OK)
        return 1;
    CHECK_HIP(hipMemcpy(&flags_found, check, 4, hipMemcpyDeviceToHost));
    if (flags_found != 0) {
        fprintf(stderr, "index validator flagged %d\n", flags_found);
        return 1;
    }

    const la_status st = gdn_decode_mtp(&a, NULL);
    if (st != LA_OK) {
        fprintf(stderr, "gdn_decode_mtp: %s\n", la_status_string(st));
        return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(hout, out, nout * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hinter, inter, ninter * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hpool_after, pool, npool * 4, hipMemcpyDeviceToHost));

    const double e_out = rel_err(hout, dout, nout);
    const double e_inter = rel_err(hinter, dinter, ninter);
    double e_state = 0.0;
    int untouched_ok = 1;
    for (int s = 0; s < P; ++s) {
        const size_t off = (size_t)s * HV * tile;
        if (s == 1 || s == 2) {
            const double e = rel_err(hpool_after + off, dpool_out + off,
                                     HV * tile);
            if (!(e <= e_state))
                e_state = e;
        } else if (memcmp(hpool_after + off, hpool + off, HV * tile * 4)) {
            untouched_ok = 0;
        }
    }
    printf("library %d, rel errors: out %.3e state %.3e inter %.3e; "
           "untouched slots %s\n", la_version(), e_out, e_state, e_inter,
           untouched_ok ? "intact" : "CHANGED");
    const int ok = e_out <= 1e-4 && e_state <= 1e-4 && e_inter <= 1e-4 &&
                   untouched_ok;
    printf("%s\n", ok ? "ok" : "MISMATCH");
    return ok ? 0 : 1;
}
