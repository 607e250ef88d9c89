/*
 * gdn_oracle_body.h -- the per-head arithmetic of the CPU oracle.
 *
 * TEST INFRASTRUCTURE. Included twice by gdn_oracle.c: once with REAL = float
 * (the reference every GPU result is compared with) and once with
 * REAL = double (used only to bound the float version's own rounding error).
 * The caller defines REAL, SUFFIX, FMA, SQRT, EXP and LOG1P before including it.
 *
 * Sources, cited by page title and section:
 *   [GDN]  Yang, Kautz, Hatamizadeh, "Gated Delta Networks: Improving Mamba2
 *          with Delta Rule" (ICLR 2025): the gated delta rule, one token at a
 *          time, with L2-normalised queries and keys.
 *   [vLLM] vLLM PR "[Spec Decode][Qwen4Exp] RecoverSSM for Qwen GDN and the
 *          PLE short conv": Purpose (the fp32 replay record holds the
 *          correction, the normalised key and the gate) and Test Result (the
 *          record keeps the decay that was multiplied in; the commit replays
 *          accepted tokens forward with the same fused update, which makes the
 *          committed state equal to the native per-token state bit for bit).
 *
 * Notation. The state h of one value head is a V x K matrix stored row-major,
 * h[v*K + kk]; a key is a K-vector, a value a V-vector. For token t:
 *   q_hat = q * (1/sqrt(sum q^2 + eps)),   q_tilde = q_hat * scale
 *   k_hat = k * (1/sqrt(sum k^2 + eps))
 *   g     = exp(a)                      (a is the log-gate, g the decay)
 *   h'    = g * h                       (rounded: this is the value replay uses)
 *   u[v]  = sum_k h'[v][k] * k_hat[k]
 *   delta = beta * (v - u)              (the correction)
 *   h     = fma(delta[v], k_hat[k], h'[v][k])
 *   o[v]  = sum_k h[v][k] * q_tilde[k]  (output from the updated state)
 * Every operation is one IEEE operation in REAL, rounded to nearest even; the
 * build turns floating-point contraction off, so only the fma written out is
 * fused. Sums run in ascending index order.
 *
 * PARITY UNPINNED against the pages (they print neither formula):
 *   - raw_gate_: the decay and write strength formed from raw projections
 *     (log-gate = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b)) is the
 *     parameterisation of [GDN]-style layers, a reading; its pieces are pinned
 *     to closed forms and library identities, the choice of formula is not.
 *   - native_head_ch_ / replay_head_ch_: one decay per key channel is this
 *     build's reading of Kimi-K3 KDA, which [vLLM] Purpose names as a user of
 *     the same protocol without giving its arithmetic; the rule is pinned to
 *     its own fp64 transition-matrix form and to the scalar rule when every
 *     channel decays alike, not to anything the pages print.
 */

#define GLUE_(a, b) a##b
#define GLUE(a, b) GLUE_(a, b)

/* L2 normalisation of one vector: out = x * (1/sqrt(sum x^2 + eps)) * mul.
 * mul is 1 for keys and the attention scale for queries; when mul == 1 the
 * last multiply is exact and changes nothing. */
static void GLUE(l2norm_, SUFFIX)(int n, const REAL* x, REAL eps, REAL mul, REAL* out)
{
    REAL ssq = 0;
    for (int i = 0; i < n; ++i) ssq = ssq + x[i] * x[i];
    REAL inv = (REAL)1 / SQRT(ssq + eps);
    for (int i = 0; i < n; ++i) {
        REAL xh = x[i] * inv;
        out[i] = xh * mul;
    }
}

/*
 * The native per-token rule over one window of w tokens of one value head,
 * starting from the checkpoint S0 (never written). For each token t it
 * produces the output o[t], the replay record (delta[t], k_hat[t], g[t]) and,
 * when snaps != NULL, the state after the token, snaps[t] = S_{t+1}.
 * h, qt, kh are caller-provided work arrays (V*K, K, K elements).
 */
static void GLUE(native_head_, SUFFIX)(
    int K, int V, const REAL* S0, int w,
    const REAL* q, const REAL* k, const REAL* vv, const REAL* a, const REAL* beta,
    REAL scale, REAL eps,
    REAL* h, REAL* qt, REAL* kh,
    REAL* o, REAL* rec_delta, REAL* rec_khat, REAL* rec_g, REAL* snaps)
{
    for (long e = 0; e < (long)V * K; ++e) h[e] = S0[e];
    for (int t = 0; t < w; ++t) {
        const REAL* qv = q + (long)t * K;
        const REAL* kv = k + (long)t * K;
        const REAL* vt = vv + (long)t * V;
        GLUE(l2norm_, SUFFIX)(K, qv, eps, scale, qt);
        GLUE(l2norm_, SUFFIX)(K, kv, eps, (REAL)1, kh);
        REAL g = EXP(a[t]);
        REAL b = beta[t];
        for (int v = 0; v < V; ++v) {
            REAL* hr = h + (long)v * K;
            /* decay first; the rounded product is what both u and the update use */
            for (int kk = 0; kk < K; ++kk) hr[kk] = hr[kk] * g;
            REAL u = 0;
            for (int kk = 0; kk < K; ++kk) u = u + hr[kk] * kh[kk];
            REAL d = b * (vt[v] - u);
            for (int kk = 0; kk < K; ++kk) hr[kk] = FMA(d, kh[kk], hr[kk]);
            REAL ov = 0;
            for (int kk = 0; kk < K; ++kk) ov = ov + hr[kk] * qt[kk];
            o[(long)t * V + v] = ov;
            rec_delta[(long)t * V + v] = d;
        }
        for (int kk = 0; kk < K; ++kk) rec_khat[(long)t * K + kk] = kh[kk];
        rec_g[t] = g;
        if (snaps)
            for (long e = 0; e < (long)V * K; ++e) snaps[(long)t * V * K + e] = h[e];
    }
}

/* Replay of n recorded tokens onto h in place: the commit update,
 * h[v][k] = fma(delta_t[v], k_hat_t[k], h[v][k] * g_t), for t = 0..n-1. */
static void GLUE(replay_head_, SUFFIX)(
    int K, int V, REAL* h, int n,
    const REAL* rec_delta, const REAL* rec_khat, const REAL* rec_g)
{
    for (int t = 0; t < n; ++t) {
        const REAL* d = rec_delta + (long)t * V;
        const REAL* kh = rec_khat + (long)t * K;
        REAL g = rec_g[t];
        for (int v = 0; v < V; ++v)
            for (int kk = 0; kk < K; ++kk) {
                REAL decayed = h[(long)v * K + kk] * g;
                h[(long)v * K + kk] = FMA(d[v], kh[kk], decayed);
            }
    }
}


/*
 * The per-key-channel decay variant (a reading of Kimi-K3 KDA: [vLLM] Purpose
 * names it as a user of the same record-and-replay protocol but the pages give
 * none of its arithmetic; the reading taken is the gated delta rule with the
 * scalar decay replaced by one decay per key channel). For token t the log-decay is a
 * K-vector a_t and alpha_t[k] = exp(a_t[k]); then
 *   h'[v][k] = h[v][k] * alpha_t[k]      (rounded; the value replay uses)
 *   u, delta, the update and o as in native_head above,
 * and the record is (delta[t], k_hat[t], alpha_t). With alpha_t[k] equal for
 * every k this is native_head exactly. al is a K-element work array.
 */
static void GLUE(native_head_ch_, SUFFIX)(
    int K, int V, const REAL* S0, int w,
    const REAL* q, const REAL* k, const REAL* vv, const REAL* a, const REAL* beta,
    REAL scale, REAL eps,
    REAL* h, REAL* qt, REAL* kh, REAL* al,
    REAL* o, REAL* rec_delta, REAL* rec_khat, REAL* rec_alpha, REAL* snaps)
{
    for (long e = 0; e < (long)V * K; ++e) h[e] = S0[e];
    for (int t = 0; t < w; ++t) {
        const REAL* qv = q + (long)t * K;
        const REAL* kv = k + (long)t * K;
        const REAL* vt = vv + (long)t * V;
        GLUE(l2norm_, SUFFIX)(K, qv, eps, scale, qt);
        GLUE(l2norm_, SUFFIX)(K, kv, eps, (REAL)1, kh);
        for (int kk = 0; kk < K; ++kk) al[kk] = EXP(a[(long)t * K + kk]);
        REAL b = beta[t];
        for (int v = 0; v < V; ++v) {
            REAL* hr = h + (long)v * K;
            for (int kk = 0; kk < K; ++kk) hr[kk] = hr[kk] * al[kk];
            REAL u = 0;
            for (int kk = 0; kk < K; ++kk) u = u + hr[kk] * kh[kk];
            REAL d = b * (vt[v] - u);
            for (int kk = 0; kk < K; ++kk) hr[kk] = FMA(d, kh[kk], hr[kk]);
            REAL ov = 0;
            for (int kk = 0; kk < K; ++kk) ov = ov + hr[kk] * qt[kk];
            o[(long)t * V + v] = ov;
            rec_delta[(long)t * V + v] = d;
        }
        for (int kk = 0; kk < K; ++kk) {
            rec_khat[(long)t * K + kk] = kh[kk];
            rec_alpha[(long)t * K + kk] = al[kk];
        }
        if (snaps)
            for (long e = 0; e < (long)V * K; ++e) snaps[(long)t * V * K + e] = h[e];
    }
}

/* Replay of n per-channel-decay records:
 * h[v][k] = fma(delta_t[v], k_hat_t[k], h[v][k] * alpha_t[k]), t = 0..n-1. */
static void GLUE(replay_head_ch_, SUFFIX)(
    int K, int V, REAL* h, int n,
    const REAL* rec_delta, const REAL* rec_khat, const REAL* rec_alpha)
{
    for (int t = 0; t < n; ++t) {
        const REAL* d = rec_delta + (long)t * V;
        const REAL* kh = rec_khat + (long)t * K;
        const REAL* al = rec_alpha + (long)t * K;
        for (int v = 0; v < V; ++v)
            for (int kk = 0; kk < K; ++kk) {
                REAL decayed = h[(long)v * K + kk] * al[kk];
                h[(long)v * K + kk] = FMA(d[v], kh[kk], decayed);
            }
    }
}

/* Gates from the raw per-token projections a, b of one value head with that
 * head's parameters A_log, dt_bias. The pages give no formula for this step;
 * the reading taken is the decay parameterisation used with Gated DeltaNet
 * layers [GDN]:
 *   x = a + dt_bias,  softplus(x) = x if x > 20, else log(1 + exp(x))
 *   log-gate = -exp(A_log) * softplus(x)      (the decay is exp(log-gate))
 *   beta     = 1 / (1 + exp(-b))
 * One IEEE operation per step, in the order written. */
static void GLUE(raw_gate_, SUFFIX)(REAL a, REAL b, REAL A_log, REAL dt_bias,
                                    REAL* log_gate, REAL* beta)
{
    REAL x = a + dt_bias;
    REAL sp = x > (REAL)20 ? x : LOG1P(EXP(x));
    REAL rate = EXP(A_log);
    *log_gate = -(rate * sp);
    *beta = (REAL)1 / ((REAL)1 + EXP(-b));
}

#undef GLUE
#undef GLUE_
