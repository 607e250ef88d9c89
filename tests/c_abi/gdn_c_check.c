/*
 * gdn_c_check.c -- drives libgdnreplay.so from plain C99 through the C ABI of
 * include/gdn_replay.h, with device memory from the HIP runtime's C API only
 * (no Python, no PyTorch), and checks the results against the CPU oracle
 * (oracle/libgdn_oracle.so: the native per-token gated delta rule that keeps
 * every state).
 *
 * TEST INFRASTRUCTURE: built by __graft_entry__.build(), run by
 * tests/test_c_abi_gpu.py on a GPU.
 *
 * One layer, three rows (the third is graph padding: null slot, empty
 * window), 4 value heads reading 2 key heads, record capacity 4:
 *   gdn_verify, then gdn_commit_all_layers in place.
 * Checks (vLLM PR "[Spec Decode][Qwen4Exp] RecoverSSM for Qwen GDN and the
 * PLE short conv", Purpose and Test Plan): outputs and committed states within
 * 1e-5 normwise of the oracle, slots no row commits to bit-identical, nothing
 * written for the padding row, no device row error.
 * Exit status 0 on success; prints one line with the errors.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gdn_replay.h"

/* oracle/libgdn_oracle.so */
int gdno_native_heads_f32(int nheads, int K, int V, int T, const float* S0, const int* w,
                          const float* q, const float* k, const float* v, const float* a,
                          const float* beta, float scale, float eps, float* o, float* rec_delta,
                          float* rec_khat, float* rec_g, float* snaps, const int* keep, float* kept,
                          int nkeep, int nthreads);
void gdno_bf16_to_f32(long n, const uint16_t* in, float* out);
void gdno_f32_to_bf16_rne(long n, const float* in, uint16_t* out);

#define D 128
#define HV 4
#define HK 2
#define T 4
#define NSLOTS 5
#define NREC 3
#define ROWS 3
#define NTOK 8
#define HEAD (D * D)

#define CHECK_HIP(x)                                                              \
    do {                                                                          \
        hipError_t e_ = (x);                                                      \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
            return 2;                                                             \
        }                                                                         \
    } while (0)

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static float uni(float lo, float hi) /* xorshift64*, uniform in [lo, hi) */
{
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return lo + (hi - lo) * (float)((rng * 0x2545f4914f6cdd1dull) >> 40) / 16777216.0f;
}

static double normwise(const float* x, const float* y, long n)
{
    double num = 0, den = 0;
    long i;
    for (i = 0; i < n; ++i) {
        double d = fabs((double)x[i] - (double)y[i]), m = fabs((double)y[i]);
        if (!(d <= num)) num = d;   /* a NaN in x wins */
        if (m > den) den = m;
    }
    return den > 0 ? num / den : num;
}

int main(void)
{
    const int slot[ROWS] = {3, 0, -1}, rec[ROWS] = {0, 1, 2};
    const int ts[ROWS] = {0, 4, 7}, win[ROWS] = {4, 3, 0}, nacc[ROWS] = {3, 1, 0};
    const long n_state = (long)NSLOTS * HV * HEAD, n_qk = (long)NTOK * HK * D;
    const long n_v = (long)NTOK * HV * D, n_g = (long)NTOK * HV, n_out = (long)NTOK * HV * D;
    const int64_t rec_stride = gdn_rec_stride(T);
    const long n_rec = (long)NREC * HV * rec_stride;
    int b, h, t, dev = 0;
    /* the shapes the kernels and their grids assume, checked on the host */
    for (b = 0; b < ROWS; ++b) {
        if (slot[b] >= NSLOTS || rec[b] < 0 || rec[b] >= NREC || win[b] < 0 || win[b] > T ||
            ts[b] < 0 || ts[b] + win[b] > NTOK || nacc[b] < 0 || nacc[b] > win[b]) {
            fprintf(stderr, "bad row %d\n", b);
            return 3;
        }
    }
    if (rec_stride < (int64_t)(2 * T * D + T)) return 3;

    float* S = malloc(sizeof(float) * n_state);
    float* S_after = malloc(sizeof(float) * n_state);
    float* qf = malloc(sizeof(float) * n_qk);
    float* kf = malloc(sizeof(float) * n_qk);
    float* vf = malloc(sizeof(float) * n_v);
    uint16_t* qb = malloc(sizeof(uint16_t) * n_qk);
    uint16_t* kb = malloc(sizeof(uint16_t) * n_qk);
    uint16_t* vb = malloc(sizeof(uint16_t) * n_v);
    float* a = malloc(sizeof(float) * n_g);
    float* beta = malloc(sizeof(float) * n_g);
    float* out = malloc(sizeof(float) * n_out);
    if (!S || !S_after || !qf || !kf || !vf || !qb || !kb || !vb || !a || !beta || !out) return 4;
    {
        long i;
        for (i = 0; i < n_state; ++i) S[i] = uni(-0.1f, 0.1f);
        for (i = 0; i < n_qk; ++i) { qf[i] = uni(-1.f, 1.f); kf[i] = uni(-1.f, 1.f); }
        for (i = 0; i < n_v; ++i) vf[i] = uni(-1.f, 1.f);
        for (i = 0; i < n_g; ++i) { a[i] = uni(-2.f, 0.f); beta[i] = uni(0.f, 1.f); }
        for (i = 0; i < n_out; ++i) out[i] = NAN;
    }
    gdno_f32_to_bf16_rne(n_qk, qf, qb);
    gdno_f32_to_bf16_rne(n_qk, kf, kb);
    gdno_f32_to_bf16_rne(n_v, vf, vb);
    gdno_bf16_to_f32(n_qk, qb, qf);   /* the values both sides see */
    gdno_bf16_to_f32(n_qk, kb, kf);
    gdno_bf16_to_f32(n_v, vb, vf);

    /* ---- device buffers (HIP runtime C API) ---- */
    void *dS, *dRec, *dq, *dk, *dv, *da, *db, *dout, *dslot, *drec, *dts, *dwin, *dn, *derr;
    CHECK_HIP(hipSetDevice(dev));
    CHECK_HIP(hipMalloc(&dS, sizeof(float) * n_state));
    CHECK_HIP(hipMalloc(&dRec, sizeof(float) * n_rec));
    CHECK_HIP(hipMalloc(&dq, sizeof(uint16_t) * n_qk));
    CHECK_HIP(hipMalloc(&dk, sizeof(uint16_t) * n_qk));
    CHECK_HIP(hipMalloc(&dv, sizeof(uint16_t) * n_v));
    CHECK_HIP(hipMalloc(&da, sizeof(float) * n_g));
    CHECK_HIP(hipMalloc(&db, sizeof(float) * n_g));
    CHECK_HIP(hipMalloc(&dout, sizeof(float) * n_out));
    CHECK_HIP(hipMalloc(&dslot, sizeof(int) * ROWS));
    CHECK_HIP(hipMalloc(&drec, sizeof(int) * ROWS));
    CHECK_HIP(hipMalloc(&dts, sizeof(int) * ROWS));
    CHECK_HIP(hipMalloc(&dwin, sizeof(int) * ROWS));
    CHECK_HIP(hipMalloc(&dn, sizeof(int) * ROWS));
    CHECK_HIP(hipMalloc(&derr, sizeof(int)));
    CHECK_HIP(hipMemcpy(dS, S, sizeof(float) * n_state, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(dRec, 0, sizeof(float) * n_rec));
    CHECK_HIP(hipMemcpy(dq, qb, sizeof(uint16_t) * n_qk, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dk, kb, sizeof(uint16_t) * n_qk, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dv, vb, sizeof(uint16_t) * n_v, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(da, a, sizeof(float) * n_g, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(db, beta, sizeof(float) * n_g, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dout, out, sizeof(float) * n_out, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dslot, slot, sizeof(int) * ROWS, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(drec, rec, sizeof(int) * ROWS, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dts, ts, sizeof(int) * ROWS, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dwin, win, sizeof(int) * ROWS, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dn, nacc, sizeof(int) * ROWS, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(derr, 0, sizeof(int)));

    /* ---- the C ABI ---- */
    gdn_pools pools;
    memset(&pools, 0, sizeof pools);
    pools.num_layers = 1; pools.num_v_heads = HV; pools.num_k_heads = HK;
    pools.head_k_dim = D; pools.head_v_dim = D; pools.state_dtype = GDN_STATE_F32;
    pools.num_state_slots = NSLOTS; pools.num_rec_slots = NREC; pools.rec_tokens = T;
    pools.record_kind = GDN_RECORD_CORRECTION;
    pools.state[0] = dS; pools.rec[0] = (float*)dRec;
    gdn_verify_io io;
    memset(&io, 0, sizeof io);
    io.q = (const uint16_t*)dq; io.q_tok_stride = HK * D; io.q_head_stride = D;
    io.k = (const uint16_t*)dk; io.k_tok_stride = HK * D; io.k_head_stride = D;
    io.v = (const uint16_t*)dv; io.v_tok_stride = HV * D; io.v_head_stride = D;
    io.a = (const float*)da; io.b = (const float*)db; io.gate_tok_stride = HV;
    io.out = dout; io.out_tok_stride = HV * D; io.out_head_stride = D;
    io.num_tokens = NTOK; io.scale = 1.0f; io.gate_mode = GDN_GATE_LOG; io.out_dtype = GDN_OUT_F32;
    int32_t st = gdn_verify(&pools, 0, ROWS, dslot, drec, dts, dwin, NULL, &io, derr, NULL);
    if (st != GDN_OK) { fprintf(stderr, "gdn_verify: %s\n", gdn_status_string(st)); return 5; }
    st = gdn_commit_all_layers(&pools, ROWS, dslot, dslot, drec, dn, NULL, NULL, derr, NULL);
    if (st != GDN_OK) { fprintf(stderr, "gdn_commit_all_layers: %s\n", gdn_status_string(st)); return 5; }
    CHECK_HIP(hipDeviceSynchronize());
    int err = -1;
    CHECK_HIP(hipMemcpy(&err, derr, sizeof(int), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(S_after, dS, sizeof(float) * n_state, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(out, dout, sizeof(float) * n_out, hipMemcpyDeviceToHost));

    /* ---- the oracle, head by head ---- */
    double e_out = 0, e_state = 0;
    int bad = err != 0;
    float q1[T * D], k1[T * D], v1[T * D], a1[T], b1[T], o1[T * D], rd[T * D], rk[T * D], rg[T];
    float* kept = malloc(sizeof(float) * HEAD);
    if (!kept) return 4;
    for (b = 0; b < ROWS; ++b) {
        if (slot[b] < 0 || win[b] == 0) continue;
        for (h = 0; h < HV; ++h) {
            const int hk = h / (HV / HK);
            memset(q1, 0, sizeof q1); memset(k1, 0, sizeof k1); memset(v1, 0, sizeof v1);
            memset(a1, 0, sizeof a1); memset(b1, 0, sizeof b1);
            for (t = 0; t < win[b]; ++t) {
                const long tok = ts[b] + t;
                memcpy(q1 + t * D, qf + (tok * HK + hk) * D, sizeof(float) * D);
                memcpy(k1 + t * D, kf + (tok * HK + hk) * D, sizeof(float) * D);
                memcpy(v1 + t * D, vf + (tok * HV + h) * D, sizeof(float) * D);
                a1[t] = a[tok * HV + h];
                b1[t] = beta[tok * HV + h];
            }
            const float* S0 = S + ((long)slot[b] * HV + h) * HEAD;
            const int keep = nacc[b];
            if (gdno_native_heads_f32(1, D, D, T, S0, &win[b], q1, k1, v1, a1, b1, 1.0f, 1e-6f, o1, rd,
                                      rk, rg, NULL, &keep, kept, 1, 1) != 0)
                return 6;
            for (t = 0; t < win[b]; ++t) {
                const double e = normwise(out + ((long)(ts[b] + t) * HV + h) * D, o1 + t * D, D);
                if (!(e <= e_out)) e_out = e;
            }
            {
                const double e = normwise(S_after + ((long)slot[b] * HV + h) * HEAD, kept, HEAD);
                if (!(e <= e_state)) e_state = e;
            }
        }
    }
    if (!(e_out <= 1e-5) || !(e_state <= 1e-5)) bad = 1;
    /* slots no row commits to: bit-identical */
    {
        int s, untouched_ok = 1;
        for (s = 0; s < NSLOTS; ++s) {
            int live = 0;
            for (b = 0; b < ROWS; ++b) live |= slot[b] == s && nacc[b] > 0;
            if (!live && memcmp(S + (long)s * HV * HEAD, S_after + (long)s * HV * HEAD,
                                sizeof(float) * HV * HEAD) != 0)
                untouched_ok = 0;
        }
        if (!untouched_ok) bad = 1;
        /* the padding row's token: nothing written */
        for (h = 0; h < HV * D; ++h)
            if (!isnan(out[(long)ts[2] * HV * D + h])) { bad = 1; break; }
        printf("c-abi check: outputs rel err %.2e, committed states rel err %.2e, untouched slots %s, "
               "row errors %d: %s\n", e_out, e_state, untouched_ok ? "identical" : "CHANGED", err,
               bad ? "FAIL" : "ok");
    }
    hipFree(dS); hipFree(dRec); hipFree(dq); hipFree(dk); hipFree(dv); hipFree(da); hipFree(db);
    hipFree(dout); hipFree(dslot); hipFree(drec); hipFree(dts); hipFree(dwin); hipFree(dn); hipFree(derr);
    free(S); free(S_after); free(qf); free(kf); free(vf); free(qb); free(kb); free(vb); free(a);
    free(beta); free(out); free(kept);
    return bad;
}
