/*
 * gdn_oracle.c -- plain, slow CPU oracle for verify-and-commit replay of Gated
 * DeltaNet recurrent state under speculative (MTP) decoding.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library. The GPU library neither
 * links nor includes it, and the two share no code, header or constant.
 *
 * It is the plain definition: the native per-token gated delta rule that keeps
 * the state after every token, a literal replay of recorded tokens, and the
 * align-mode slot plan as a walk over token positions. The per-head arithmetic
 * is in gdn_oracle_body.h; this file adds the batch drivers (independent heads
 * packed one after another, an OpenMP loop over heads), the bf16 conversions
 * and the align plan.
 *
 * Sources, cited by page title and section:
 *   [vLLM] vLLM PR "[Spec Decode][Qwen4Exp] RecoverSSM for Qwen GDN and the
 *          PLE short conv": Purpose, Commits items 3 and 6, Test Plan,
 *          Test Result.
 *   [TS]   tokenspeed PR "feat: add Qwen3.5 GDN ReplaySSM": Summary,
 *          Motivation.
 *   [LMD]  lmdeploy PR #5028 (opt-in ReplaySSM): Performance test settings
 *          (16-token replay buffer, 64-token blocks, fp32 SSM state).
 *   [GDN]  Yang, Kautz, Hatamizadeh, "Gated Delta Networks" (ICLR 2025).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -shared -fPIC (no fast
 * math, IEEE denormals kept).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define REAL float
#define SUFFIX f32
#define FMA fmaf
#define SQRT sqrtf
#define EXP expf
#define LOG1P log1pf
#include "gdn_oracle_body.h"
#undef REAL
#undef SUFFIX
#undef FMA
#undef SQRT
#undef EXP
#undef LOG1P

#define REAL double
#define SUFFIX f64
#define FMA fma
#define SQRT sqrt
#define EXP exp
#define LOG1P log1p
#include "gdn_oracle_body.h"
#undef REAL
#undef SUFFIX
#undef FMA
#undef SQRT
#undef EXP
#undef LOG1P

int gdno_version(void) { return 1; }

/* ---------------------------------------------------------------------------
 * Batch drivers. Heads are independent ([GDN]: one recurrent state per value
 * head), so a batch is nheads windows packed back to back:
 *   S0[nheads][V][K], q/k[nheads][T][K], v[nheads][T][V], a/beta[nheads][T],
 *   w[nheads] (tokens to run, 0..T). Outputs o/rec_delta [nheads][T][V],
 *   rec_khat [nheads][T][K], rec_g [nheads][T]; only the first w[i] tokens of
 *   head i are written.
 *   snaps  [nheads][T][V][K] or NULL: S_1..S_w of every head.
 *   keep   [nheads][nkeep] or NULL: indices j in 0..w of states S_j to copy
 *          into kept[nheads][nkeep][V][K] (S_0 is the checkpoint itself);
 *          a negative index leaves that entry unwritten.
 * Return 0, or -1 on a bad argument.
 * ------------------------------------------------------------------------- */

#define BATCH_NATIVE(SUF, R)                                                            \
int gdno_native_heads_##SUF(int nheads, int K, int V, int T,                            \
    const R* S0, const int* w, const R* q, const R* k, const R* v,                      \
    const R* a, const R* beta, R scale, R eps,                                          \
    R* o, R* rec_delta, R* rec_khat, R* rec_g, R* snaps,                                \
    const int* keep, R* kept, int nkeep, int nthreads)                                  \
{                                                                                       \
    if (nheads < 0 || K < 1 || V < 1 || T < 1 || nkeep < 0) return -1;                  \
    for (int i = 0; i < nheads; ++i) if (w[i] < 0 || w[i] > T) return -1;               \
    if (keep)                                                                           \
        for (long i = 0; i < (long)nheads * nkeep; ++i)                                 \
            if (keep[i] > w[i / (nkeep ? nkeep : 1)]) return -1;                        \
    const long VK = (long)V * K;                                                        \
    int bad = 0;                                                                        \
    _Pragma("omp parallel num_threads(nthreads > 0 ? nthreads : 1)")                    \
    {                                                                                   \
        R* h = (R*)malloc(sizeof(R) * VK);                                              \
        R* qt = (R*)malloc(sizeof(R) * K);                                              \
        R* kh = (R*)malloc(sizeof(R) * K);                                              \
        R* loc = (R*)malloc(sizeof(R) * VK * (T + 1));                                  \
        int ok = h && qt && kh && loc;                                                  \
        if (!ok) {                                                                      \
            _Pragma("omp atomic write") bad = 1;                                        \
        }                                                                               \
        {   /* every thread reaches the worksharing loop */                             \
            _Pragma("omp for schedule(dynamic, 4)")                                     \
            for (int i = 0; i < nheads; ++i) {                                          \
                if (!ok) continue;                                                      \
                const long tk = (long)i * T;                                            \
                /* keep every state locally: loc[0] = S_0, loc[j] = S_j */              \
                memcpy(loc, S0 + i * VK, sizeof(R) * VK);                               \
                native_head_##SUF(K, V, S0 + i * VK, w[i], q + tk * K, k + tk * K,      \
                    v + tk * V, a + tk, beta + tk, scale, eps, h, qt, kh,               \
                    o + tk * V, rec_delta + tk * V, rec_khat + tk * K, rec_g + tk,      \
                    loc + VK);                                                          \
                if (snaps)                                                              \
                    memcpy(snaps + tk * VK, loc + VK, sizeof(R) * VK * w[i]);           \
                if (keep)                                                               \
                    for (int j = 0; j < nkeep; ++j) {                                   \
                        int s = keep[(long)i * nkeep + j];                              \
                        if (s >= 0)                                                     \
                            memcpy(kept + ((long)i * nkeep + j) * VK, loc + s * VK,     \
                                   sizeof(R) * VK);                                     \
                    }                                                                   \
            }                                                                           \
        }                                                                               \
        free(h); free(qt); free(kh); free(loc);                                         \
    }                                                                                   \
    return bad ? -1 : 0;                                                                \
}

BATCH_NATIVE(f32, float)
BATCH_NATIVE(f64, double)

/* The per-key-channel decay variant, batched like gdno_native_heads: a and
 * rec_alpha are [nheads][T][K] (a log-decay and a decay per key channel);
 * everything else as there. */
#define BATCH_NATIVE_CH(SUF, R)                                                         \
int gdno_native_heads_ch_##SUF(int nheads, int K, int V, int T,                         \
    const R* S0, const int* w, const R* q, const R* k, const R* v,                      \
    const R* a, const R* beta, R scale, R eps,                                          \
    R* o, R* rec_delta, R* rec_khat, R* rec_alpha, R* snaps,                            \
    const int* keep, R* kept, int nkeep, int nthreads)                                  \
{                                                                                       \
    if (nheads < 0 || K < 1 || V < 1 || T < 1 || nkeep < 0) return -1;                  \
    for (int i = 0; i < nheads; ++i) if (w[i] < 0 || w[i] > T) return -1;               \
    if (keep)                                                                           \
        for (long i = 0; i < (long)nheads * nkeep; ++i)                                 \
            if (keep[i] > w[i / (nkeep ? nkeep : 1)]) return -1;                        \
    const long VK = (long)V * K;                                                        \
    int bad = 0;                                                                        \
    _Pragma("omp parallel num_threads(nthreads > 0 ? nthreads : 1)")                    \
    {                                                                                   \
        R* h = (R*)malloc(sizeof(R) * VK);                                              \
        R* qt = (R*)malloc(sizeof(R) * K);                                              \
        R* kh = (R*)malloc(sizeof(R) * K);                                              \
        R* al = (R*)malloc(sizeof(R) * K);                                              \
        R* loc = (R*)malloc(sizeof(R) * VK * (T + 1));                                  \
        int ok = h && qt && kh && al && loc;                                            \
        if (!ok) {                                                                      \
            _Pragma("omp atomic write") bad = 1;                                        \
        }                                                                               \
        {                                                                               \
            _Pragma("omp for schedule(dynamic, 4)")                                     \
            for (int i = 0; i < nheads; ++i) {                                          \
                if (!ok) continue;                                                      \
                const long tk = (long)i * T;                                            \
                memcpy(loc, S0 + i * VK, sizeof(R) * VK);                               \
                native_head_ch_##SUF(K, V, S0 + i * VK, w[i], q + tk * K, k + tk * K,   \
                    v + tk * V, a + tk * K, beta + tk, scale, eps, h, qt, kh, al,       \
                    o + tk * V, rec_delta + tk * V, rec_khat + tk * K,                  \
                    rec_alpha + tk * K, loc + VK);                                      \
                if (snaps)                                                              \
                    memcpy(snaps + tk * VK, loc + VK, sizeof(R) * VK * w[i]);           \
                if (keep)                                                               \
                    for (int j = 0; j < nkeep; ++j) {                                   \
                        int s = keep[(long)i * nkeep + j];                              \
                        if (s >= 0)                                                     \
                            memcpy(kept + ((long)i * nkeep + j) * VK, loc + s * VK,     \
                                   sizeof(R) * VK);                                     \
                    }                                                                   \
            }                                                                           \
        }                                                                               \
        free(h); free(qt); free(kh); free(al); free(loc);                               \
    }                                                                                   \
    return bad ? -1 : 0;                                                                \
}

BATCH_NATIVE_CH(f32, float)
BATCH_NATIVE_CH(f64, double)

/* Replay n[i] per-channel-decay records of head i onto S[i] in place. */
int gdno_replay_heads_ch_f32(int nheads, int K, int V, int T, float* S, const int* n,
                             const float* rec_delta, const float* rec_khat,
                             const float* rec_alpha, int nthreads)
{
    if (nheads < 0 || K < 1 || V < 1 || T < 1) return -1;
    for (int i = 0; i < nheads; ++i) if (n[i] < 0 || n[i] > T) return -1;
    const long VK = (long)V * K;
    #pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads > 0 ? nthreads : 1)
    for (int i = 0; i < nheads; ++i) {
        const long tk = (long)i * T;
        replay_head_ch_f32(K, V, S + i * VK, n[i], rec_delta + tk * V, rec_khat + tk * K,
                           rec_alpha + tk * K);
    }
    return 0;
}

/* Gates from raw inputs for n (token, value head) entries laid out
 * [tokens][HV] (head fastest): entry i uses A_log[i % hv], dt_bias[i % hv].
 * Writes the log-gate (the decay is exp of it) and beta. Return 0, or -1 on
 * a bad argument. */
#define BATCH_RAW_GATES(SUF, R)                                                        \
int gdno_raw_gates_##SUF(long n, int hv, const R* a, const R* b, const R* A_log,        \
                         const R* dt_bias, R* log_gate, R* beta)                        \
{                                                                                       \
    if (n < 0 || hv < 1) return -1;                                                     \
    for (long i = 0; i < n; ++i)                                                        \
        raw_gate_##SUF(a[i], b[i], A_log[i % hv], dt_bias[i % hv], log_gate + i,        \
                       beta + i);                                                       \
    return 0;                                                                           \
}

BATCH_RAW_GATES(f32, float)
BATCH_RAW_GATES(f64, double)

/* Replay n[i] recorded tokens of head i onto S[i] in place ([vLLM] Test
 * Result: h = fma(correction, key, h * decay), token by token). */
int gdno_replay_heads_f32(int nheads, int K, int V, int T, float* S, const int* n,
                          const float* rec_delta, const float* rec_khat,
                          const float* rec_g, int nthreads)
{
    if (nheads < 0 || K < 1 || V < 1 || T < 1) return -1;
    for (int i = 0; i < nheads; ++i) if (n[i] < 0 || n[i] > T) return -1;
    const long VK = (long)V * K;
    #pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads > 0 ? nthreads : 1)
    for (int i = 0; i < nheads; ++i) {
        const long tk = (long)i * T;
        replay_head_f32(K, V, S + i * VK, n[i], rec_delta + tk * V, rec_khat + tk * K,
                        rec_g + tk);
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * bf16 <-> fp32. A bf16 value is the top 16 bits of an fp32 value, so the
 * widening is exact. Narrowing rounds to nearest, ties to even ([vLLM] Test
 * Plan: a bf16 recurrent state is rounded once, at the commit's write). NaN
 * stays NaN (quiet bit set).
 * ------------------------------------------------------------------------- */
void gdno_bf16_to_f32(long n, const uint16_t* in, float* out)
{
    for (long i = 0; i < n; ++i) {
        uint32_t u = (uint32_t)in[i] << 16;
        memcpy(out + i, &u, 4);
    }
}

void gdno_f32_to_bf16_rne(long n, const float* in, uint16_t* out)
{
    for (long i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, in + i, 4);
        if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
            out[i] = (uint16_t)((u >> 16) | 0x0040u);
            continue;
        }
        uint32_t lower = u & 0xffffu;           /* the bits that are dropped */
        uint32_t upper = u >> 16;
        if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1;
        out[i] = (uint16_t)upper;
    }
}

/* ---------------------------------------------------------------------------
 * Align-mode slot plan, as a walk over token positions.
 *
 * Row b has a checkpoint covering its first p0 tokens and n accepted tokens at
 * positions p0 .. p0+n-1. Block c of the row's table holds tokens
 * [c*block, (c+1)*block). A state that covers m tokens lives in the block
 * holding its last token, column (m-1)/block:
 *   - the checkpoint (m = p0) is read from src = table[(p0-1)/block];
 *   - the final state (m = p0+n) goes to dst = table[(p0+n-1)/block]; a window
 *     that ends exactly on a block boundary therefore stays in the block of
 *     its last token, not the next column ([vLLM] Commits item 3);
 *   - a state after t < n accepted tokens whose m = p0+t is a multiple of
 *     block is the block-boundary state ([vLLM] Purpose: align mode also
 *     writes it); it goes to table[(m-1)/block], recorded as bnd_len = t.
 * When the boundary and final state would share a slot only the final state
 * is written ([vLLM] Commits item 6). n = 0 writes nothing: dst = -1.
 *
 * Error bits (the library's documented row-error values): 4 = n out of range,
 * 8 = more than one boundary in the window, 16 = block-table column out of
 * range or an empty (negative) table entry where a slot is needed, 64 = p0 < 1.
 * A row with an error gets src = dst = bnd_slot = -1, bnd_len = 0.
 * Returns the OR of all row errors.
 * ------------------------------------------------------------------------- */
int gdno_align_plan(int rows, const int* p0, const int* n, const int* table,
                    long table_row_stride, int table_cols, int block, int max_n,
                    int* src, int* dst, int* bnd_len, int* bnd_slot, int* row_err)
{
    int all = 0;
    for (int b = 0; b < rows; ++b) {
        const int* tb = table + (long)b * table_row_stride;
        int err = 0;
        int s = -1, d = -1, bl = 0, bs = -1, nb = 0;
        if (p0[b] < 1) err |= 64;
        if (n[b] < 0 || n[b] > max_n) err |= 4;
        if (!err) {
            long col = ((long)p0[b] - 1) / block;
            if (col >= table_cols || tb[col] < 0) err |= 16;
            else s = tb[col];
        }
        if (!err) {
            for (int t = 1; t <= n[b]; ++t) {
                long m = (long)p0[b] + t;            /* tokens covered by S_t */
                long col = (m - 1) / block;
                int is_final = (t == n[b]);
                int is_bnd = (m % block) == 0;
                if (!is_final && !is_bnd) continue;
                if (col >= table_cols || tb[col] < 0) { err |= 16; break; }
                if (is_final) {
                    d = tb[col];
                } else {
                    if (nb++) { err |= 8; break; }
                    bl = t;
                    bs = tb[col];
                }
            }
            if (!err && bl > 0 && bs == d) { bl = 0; bs = -1; }
        }
        if (err) { s = -1; d = -1; bl = 0; bs = -1; }
        src[b] = s; dst[b] = d; bnd_len[b] = bl; bnd_slot[b] = bs;
        if (row_err) row_err[b] = err;
        all |= err;
    }
    return all;
}
