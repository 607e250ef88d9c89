/*
 * gdn_replay.h -- C ABI of the MI355X (gfx950) verify-and-commit library for
 * Gated DeltaNet recurrent state under speculative (MTP) decoding.
 *
 * The method, cited by page title and section:
 *   [vLLM] vLLM PR "[Spec Decode][Qwen4Exp] RecoverSSM for Qwen GDN and the
 *          PLE short conv" -- Purpose (verify from a read-only checkpoint,
 *          fp32 per-token record of correction, normalised key and gate;
 *          commit after sampling replays only the accepted tokens and writes
 *          the state once, plus the block-boundary state in align mode;
 *          padding rows have a null slot and a zero-length window), Commits
 *          items 2, 3 and 6 (strided q/k/v views written straight into the
 *          layer output; a window ending on a boundary stays in its last
 *          token's block; final folds before boundary folds), Test Plan
 *          (bf16 state; malformed-input rejection), Test Result (the commit
 *          replays h = fma(correction, key, h * decay) and equals the native
 *          per-token state bit for bit).
 *   [TS]   tokenspeed PR "feat: add Qwen3.5 GDN ReplaySSM" -- Summary and
 *          Implementation (one all-layer commit launch; layer-indexed state
 *          and replay pools; a cooperative 4-warp block per 128x128 head).
 *   [LMD]  lmdeploy PR #5028 (opt-in ReplaySSM) -- Performance test settings
 *          (16-token replay buffer; 64-token blocks; fp32 SSM state) and the
 *          file list (cursor commits and checkpoint flushing).
 *   [GDN]  Yang, Kautz, Hatamizadeh, "Gated Delta Networks" (ICLR 2025): the
 *          per-token gated delta rule.
 *
 * Per token t of one value head (K = V = 128, all fp32):
 *   k_hat = k / sqrt(|k|^2 + 1e-6),  q_tilde = scale * q / sqrt(|q|^2 + 1e-6)
 *   g = exp(a)  (a = log-gate; see gdn_verify_io for the raw-input gating),
 *   h' = g * h
 *   delta = beta * (v - h' k_hat),  h = fma(delta, k_hat^T, h')
 *   o_t = h q_tilde
 * Value head hv reads key head hv / (HV / HK).
 *
 * Conventions for every entry point:
 *   - All pointers named "device" are HIP device memory owned by the caller.
 *     The library allocates nothing and keeps no pointer after returning.
 *   - gdn_pools and gdn_verify_io are host structs, read during the call.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream), never synchronise the host, and are capturable in a HIP graph.
 *   - Host-checkable errors return a negative gdn_status and launch nothing.
 *   - Per-row device data out of range makes the kernel skip that row and OR
 *     a GDN_ROW_* bit into *err_flags (device int32, may be NULL). The caller
 *     clears *err_flags.
 *   - Preconditions not checked: no two live rows share a state, destination,
 *     boundary or record slot; buffers are as large as the sizes say.
 */
#ifndef GDN_REPLAY_H
#define GDN_REPLAY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 5
#define GDN_MAX_LAYERS 64      /* layers per pool set */
#define GDN_HEAD_DIM 128       /* K = V = 128 */
#define GDN_MAX_REC_TOKENS 16  /* record capacity T per row */

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = -1,    /* a required pointer is NULL */
    GDN_ERR_SHAPE = -2,   /* a size or index argument is out of range */
    GDN_ERR_DTYPE = -3,   /* unsupported state or output dtype */
    GDN_ERR_ALIGN = -4,   /* a pointer or stride breaks the 16-byte rule */
    GDN_ERR_LAUNCH = -5   /* the HIP launch failed */
} gdn_status;

typedef enum { GDN_STATE_F32 = 0, GDN_STATE_BF16 = 1 } gdn_state_dtype;
typedef enum { GDN_GATE_LOG = 0, GDN_GATE_RAW = 1, GDN_GATE_CHANNEL = 2 } gdn_gate_mode;
typedef enum { GDN_RECORD_CORRECTION = 0, GDN_RECORD_PAYLOAD = 1, GDN_RECORD_CHANNEL = 2 }
    gdn_record_kind;
typedef enum { GDN_OUT_F32 = 0, GDN_OUT_BF16 = 1 } gdn_out_dtype;

/* Device row-error bits (OR'ed into *err_flags). */
enum {
    GDN_ROW_SLOT = 1,    /* a state / destination slot >= num_state_slots */
    GDN_ROW_WIN = 2,     /* window: w < 0, rec_base < 0, rec_base + w > T, or tokens out of range */
    GDN_ROW_N = 4,       /* accepted count < 0 or > T, or n > 0 with a null destination */
    GDN_ROW_BND = 8,     /* boundary length not 0 and not in (0, n), bad boundary slot,
                            or (plan) more than one block boundary inside the window */
    GDN_ROW_TABLE = 16,  /* (plan) block-table column out of range or empty where needed */
    GDN_ROW_REC = 32,    /* record slot < 0 or >= num_rec_slots for a live row */
    GDN_ROW_POS = 64,    /* (plan) num_computed < 1 */
    GDN_ROW_ALIAS = 128  /* (slot check) a slot shared between live rows; see gdn_check_slots */
};

/*
 * Layer-indexed state and record pools ([TS] Implementation; [vLLM] Purpose).
 *
 * state[l]: device, layer l's checkpoint pool, [num_state_slots][HV][V][K],
 *   K contiguous, fp32 or bf16 per state_dtype. 16-byte aligned.
 * rec[l]: device, layer l's record pool, [num_rec_slots][HV][rec_stride]
 *   floats with rec_stride = gdn_record_stride(rec_tokens, record_kind).
 *   Position p of the window (ring position in ring mode) is at index p of
 *   each field. 16-byte aligned. Records live only from a step's verify to
 *   its commit. The block of one (record slot, value head) is
 *   GDN_RECORD_CORRECTION ([vLLM] Purpose), all fp32:
 *     delta[T][V] | k_hat[T][K] | gate[T] | padding to 4 floats;
 *   GDN_RECORD_PAYLOAD (the raw-input record of [TS] Motivation: the commit
 *     recomputes the corrections, reductions included):
 *     k[T][K] bf16 (the key head's raw key) | v[T][V] bf16 | gate[T] fp32 |
 *     beta[T] fp32 | padding to 16 bytes.
 *   GDN_RECORD_CHANNEL (a reading of Kimi-K3 KDA, which [vLLM] Purpose names
 *     as a user of the same protocol without giving its arithmetic: the
 *     scalar decay becomes one decay per key channel), fp32:
 *     delta[T][V] | k_hat[T][K] | alpha[T][K]; it goes with gate_mode
 *     GDN_GATE_CHANNEL and the commit replays
 *     h[v][k] = fma(delta_t[v], k_hat_t[k], h[v][k] * alpha_t[k]).
 *   The payload record cannot serve ring mode (pending records would need
 *   their corrections), so verify rejects a rec_base with it.
 */
typedef struct gdn_pools {
    int32_t num_layers;       /* 1..GDN_MAX_LAYERS */
    int32_t num_v_heads;      /* HV >= 1 */
    int32_t num_k_heads;      /* HK >= 1, HV % HK == 0 */
    int32_t head_k_dim;       /* must be 128 */
    int32_t head_v_dim;       /* must be 128 */
    int32_t state_dtype;      /* gdn_state_dtype */
    int32_t num_state_slots;  /* >= 1 */
    int32_t num_rec_slots;    /* >= 1 */
    int32_t rec_tokens;       /* T, 1..GDN_MAX_REC_TOKENS */
    int32_t record_kind;      /* gdn_record_kind */
    void* state[GDN_MAX_LAYERS];
    float* rec[GDN_MAX_LAYERS];
} gdn_pools;

/*
 * Per-token inputs and outputs of one layer's verify ([vLLM] Commits item 2:
 * the verify reads strided q/k/v views of the short-conv output and writes
 * straight into the layer output). Strides are in elements; the innermost
 * (feature) dimension is contiguous.
 *   q, k: device bf16 bits, [tokens][HK][K];  v: device bf16 bits, [tokens][HV][V].
 *     Base pointers 16-byte aligned, strides multiples of 8 elements.
 *   a, b: device fp32 [tokens][HV] (head stride 1, token stride gate_tok_stride).
 *     gate_mode GDN_GATE_LOG: a is the log-gate (decay g = exp(a)) and b the
 *       write strength beta.
 *     gate_mode GDN_GATE_RAW: a and b are the layer's raw gate projections and
 *       the gates are formed in the kernel with the per-head parameters
 *       A_log, dt_bias (device fp32 [HV], 4-byte aligned):
 *         g = exp(-exp(A_log[h]) * softplus(a + dt_bias[h])),  beta = sigmoid(b),
 *       softplus(x) = x for x > 20, else log(1 + exp(x)). This parameterisation
 *       is not printed on the pages; it is the decay/write-strength form used
 *       with Gated DeltaNet layers ([GDN]).
 *     gate_mode GDN_GATE_CHANNEL (pools->record_kind GDN_RECORD_CHANNEL, and
 *       only then): a is one log-decay per key channel, device fp32
 *       [tokens][HV][K] at a[tok * decay_tok_stride + h * K + k] (16-byte
 *       aligned, decay_tok_stride a multiple of 4 and >= HV * K), the decay of
 *       channel k is alpha[k] = exp(a[..k]) and h' = h * alpha column by
 *       column; b is beta as in GDN_GATE_LOG.
 *     Either way the record holds the decay that was multiplied in.
 *   out: device [tokens][HV][V], fp32 (out_dtype GDN_OUT_F32; 16-byte aligned,
 *     strides multiples of 4) or bf16 bits rounded to nearest even once
 *     (GDN_OUT_BF16; 8-byte aligned, strides multiples of 4).
 *   num_tokens: rows address tokens [tok_start, tok_start + w) < num_tokens.
 *   scale: multiplies the normalised query (1 = the plain o_t = S_t q_t).
 */
typedef struct gdn_verify_io {
    const uint16_t* q;  int64_t q_tok_stride, q_head_stride;
    const uint16_t* k;  int64_t k_tok_stride, k_head_stride;
    const uint16_t* v;  int64_t v_tok_stride, v_head_stride;
    const float* a;     const float* b;  int64_t gate_tok_stride;
    void* out;          int64_t out_tok_stride, out_head_stride;
    int64_t num_tokens;
    float scale;
    int32_t gate_mode;      /* gdn_gate_mode */
    const float* A_log;     /* GDN_GATE_RAW only, else ignored */
    const float* dt_bias;   /* GDN_GATE_RAW only, else ignored */
    int32_t out_dtype;      /* gdn_out_dtype */
    int32_t reserved;       /* set to 0 */
    int64_t decay_tok_stride;  /* GDN_GATE_CHANNEL only: token stride of a, else ignored */
} gdn_verify_io;

/*
 * gdn_verify -- verify one layer's draft windows from the read-only
 * checkpoint ([vLLM] Purpose; Test Plan: checkpoint untouched).
 *
 * For each row b (all arrays device int32 [num_rows]):
 *   state_slot[b] < 0 or win_len[b] == 0: the row is padding and nothing at
 *     all is read or written for it ([vLLM] Purpose, graph padding rows).
 *   Otherwise the kernel loads S = state[layer][state_slot[b]] (bf16 widened
 *   exactly), first replays the rec_base[b] records already at positions
 *   0..rec_base-1 of record slot rec_slot[b] (ring mode, [LMD]; rec_base may
 *   be NULL = all zero), then runs tokens tok_start[b] .. tok_start[b]+w-1:
 *   writes o_t into io->out and the record (delta, k_hat, gate; or with the
 *   payload record kind k, v, gate, beta) at position rec_base + t. The
 *   state pool is never written.
 * Errors: GDN_ERR_* as in the conventions (GDN_ERR_SHAPE also when
 * num_rows * HV * 512 exceeds 2^32 - 1, the work-items one launch may hold);
 * device rows with a bad slot, window or record slot are skipped with
 * GDN_ROW_SLOT / _WIN / _REC.
 */
int32_t gdn_verify(const gdn_pools* pools, int32_t layer, int32_t num_rows,
                   const int32_t* state_slot, const int32_t* rec_slot,
                   const int32_t* tok_start, const int32_t* win_len,
                   const int32_t* rec_base, const gdn_verify_io* io,
                   int32_t* err_flags, void* stream);

/*
 * gdn_commit_all_layers -- after sampling, replay each row's accepted prefix
 * and write the state once, for every layer in one launch ([TS] Summary;
 * [vLLM] Purpose, Test Result).
 *
 * Launch shape: each (layer, row, value head) is split over several 4-wave
 * workgroups, each owning a contiguous run of the head's rows (8 KiB of
 * state: 8 workgroups of 16 rows for fp32 pools, 4 of 32 rows for bf16
 * pools; [TS] uses one 4-warp block per head, the split streams faster on
 * MI355X). For row b (device int32 arrays [num_rows]):
 *   n = n_accept[b]; if n == 0 or src_slot[b] < 0 nothing is read or written.
 *   h = state[l][src_slot[b]]; for t < n: h = fma(delta_t, k_hat_t^T, h * g_t)
 *   with the records of rec_slot[b] (per-channel decay records: h * alpha_t
 *   column by column; payload records: the correction recomputed first); the
 *   final h is written to dst_slot[b] (dst == src: in place). bf16 pools
 *   round once, to nearest even, here.
 *   Align mode (bnd_len and bnd_slot non-NULL): when 0 < bnd_len[b] < n the
 *   state after bnd_len[b] tokens is also written to bnd_slot[b], after the
 *   final state and from the same single read of the source, and not at all
 *   when bnd_slot[b] == dst_slot[b] ([vLLM] Commits item 6). Each thread
 *   reads every source element it owns before its first store and writes only
 *   those elements (a workgroup's rows are its own), so a boundary or final
 *   slot equal to the source slot is safe.
 * Launches: one, unless the grid would exceed the 2^32 - 1 work-items one
 *   launch may hold (fp32 pools: more than 2^21 (layer, row, value head)
 *   triples); then consecutive launches on `stream`, each over a run of whole
 *   layers (a launch that fails returns GDN_ERR_LAUNCH after the earlier
 *   ones have been issued). One layer's workgroups (num_rows * HV * 8, plus
 *   the conv compaction's) must fit in one launch, else GDN_ERR_SHAPE.
 * Errors: GDN_ROW_SLOT, _N, _BND, _REC for bad device rows (row skipped).
 */
int32_t gdn_commit_all_layers(const gdn_pools* pools, int32_t num_rows,
                              const int32_t* src_slot, const int32_t* dst_slot,
                              const int32_t* rec_slot, const int32_t* n_accept,
                              const int32_t* bnd_len, const int32_t* bnd_slot,
                              int32_t* err_flags, void* stream);

/*
 * Short-conv state pools for the all-layer commit ([vLLM] Purpose: the short
 * conv beside each GDN layer compacts its accepted window with the same plan;
 * Test Plan: spec conv + commit against the stock token-by-token decode).
 *
 * A causal short conv of kernel width W and dilation d keeps the last
 * L_s = (W - 1) * d inputs of every channel. Its state of one slot is
 * [L_s][C] (oldest row first, channels contiguous); decoding one token with
 * input x drops the oldest row and appends x. After a verify window the
 * commit keeps, for n accepted tokens, the last L_s rows of
 * [state rows 0..L_s-1, x_0 .. x_{n-1}].
 *
 * state[l]: device, layer l's conv pool, [num_slots][state_len][channels].
 * x[l]: device, layer l's conv inputs of this step, [num_tokens][x_tok_stride]
 *   (channels contiguous, same dtype as the state); row b's window starts at
 *   token tok_start[b] (the commit's conv_tok_start argument).
 * Bytes per state row (channels * element size) and per x token stride must be
 * multiples of 16; pointers 16-byte aligned.
 */
typedef struct gdn_conv_pools {
    int32_t num_layers;       /* 1..GDN_MAX_LAYERS */
    int32_t channels;         /* C >= 1 */
    int32_t state_len;        /* L_s, 1..GDN_MAX_CONV_STATE */
    int32_t dtype;            /* gdn_state_dtype of states and inputs */
    int32_t num_slots;        /* >= 1 */
    int32_t reserved;         /* set to 0 */
    int64_t x_tok_stride;     /* elements between consecutive tokens of x */
    int64_t num_tokens;       /* tokens addressable in x */
    void* state[GDN_MAX_LAYERS];
    const void* x[GDN_MAX_LAYERS];
} gdn_conv_pools;

#define GDN_MAX_CONV_STATE 1024

/*
 * gdn_commit_all_layers_conv -- gdn_commit_all_layers plus the short-conv
 * state compaction of the same rows, in the same single launch ([vLLM]
 * Purpose; review thread: plan, conv and state launches per group cost host
 * time, one launch over everything is preferred).
 *
 * pools may be NULL (conv states only; rec_slot is then unused) and conv may
 * be NULL (identical to gdn_commit_all_layers). With both, num_layers must
 * match. The SSM part is exactly gdn_commit_all_layers. For the conv part,
 * row b with n = n_accept[b] > 0 and src_slot[b] >= 0 writes
 *   final:    rows i = 0..L_s-1 of dst_slot[b] = row n + i of
 *             [src rows 0..L_s-1, x[tok_start[b]] .. x[tok_start[b] + n - 1]]
 *   boundary: when 0 < bnd_len[b] < n and bnd_slot[b] != dst_slot[b], rows
 *             i of bnd_slot[b] = row bnd_len[b] + i of the same sequence,
 * both formed from the source rows as they were before the call. The final
 * rows are written first, then the boundary rows, except when the final slot
 * is the source slot: the boundary rows (then in another slot) go first, since
 * the final shift overwrites source rows they are copied from. Either state
 * written over its own source slot is shifted in place (row i is written only
 * after row n + i, or bnd_len + i, has been read), so a final or boundary slot
 * equal to the source slot is safe.
 * conv_tok_start: device int32 [num_rows], needed when conv is given.
 * Errors: as gdn_commit_all_layers; GDN_ROW_SLOT for conv slots outside
 * [0, conv->num_slots), GDN_ROW_WIN for a window outside x.
 */
int32_t gdn_commit_all_layers_conv(const gdn_pools* pools, const gdn_conv_pools* conv,
                                   int32_t num_rows, const int32_t* src_slot,
                                   const int32_t* dst_slot, const int32_t* rec_slot,
                                   const int32_t* n_accept, const int32_t* bnd_len,
                                   const int32_t* bnd_slot, const int32_t* conv_tok_start,
                                   int32_t* err_flags, void* stream);

/*
 * gdn_align_plan -- align-mode slots of each row from its block table
 * ([vLLM] Purpose; Commits items 3 and 6).
 *
 * Row b has a checkpoint covering num_computed[b] = p0 >= 1 tokens and
 * n = n_accept[b] (0..max_accept) accepted tokens. A state covering m tokens
 * lives in block column (m - 1) / block_size of block_table (device int32,
 * row stride bt_row_stride elements, bt_cols columns, -1 = unallocated):
 *   src_slot = table[(p0-1)/B];  dst_slot = table[(p0+n-1)/B] (-1 if n == 0);
 *   if the window crosses a block boundary after t < n tokens ((p0+t) % B == 0)
 *   bnd_len = t and bnd_slot = table[(p0+t-1)/B] (else 0 and -1); a boundary
 *   slot equal to the final slot is dropped.
 * Outputs: device int32 [num_rows]. Rows with an error (GDN_ROW_POS, _N, _BND
 * for a second boundary, _TABLE) get all four outputs null.
 * Host errors: block_size < 1, max_accept < 0, bt_cols < 1, strides < bt_cols.
 */
int32_t gdn_align_plan(int32_t num_rows, const int32_t* num_computed,
                       const int32_t* n_accept, const int32_t* block_table,
                       int64_t bt_row_stride, int32_t bt_cols, int32_t block_size,
                       int32_t max_accept, int32_t* src_slot, int32_t* dst_slot,
                       int32_t* bnd_len, int32_t* bnd_slot, int32_t* err_flags,
                       void* stream);

/*
 * gdn_check_slots -- debug check of the slot preconditions that the hot-path
 * calls state but do not check (the check is quadratic in the rows).
 *
 * The commit's rows run concurrently; the pages' align-mode race ([vLLM]
 * Commits item 6) is one program overwriting a slot another still reads.
 * Within a row the library is safe (every thread reads its source before it
 * stores). Across rows, among the live rows (n_accept > 0 and src_slot >= 0),
 * a row's written slots are its dst_slot and, when bnd_len > 0 and
 * bnd_slot != dst_slot, its bnd_slot. For every live row that
 *   - writes a slot another live row writes, or
 *   - writes a slot another live row reads as its src_slot, or
 *   - shares its rec_slot with another live row (when rec_slot is given),
 * the kernel ORs GDN_ROW_ALIAS into *err_flags. It reads only the slot
 * arrays and writes only *err_flags.
 *
 * src_slot, dst_slot, n_accept: device int32 [num_rows]; rec_slot: device
 * int32 [num_rows] or NULL (not checked); bnd_len, bnd_slot: both device
 * int32 [num_rows] or both NULL (no boundaries); err_flags: device int32
 * (required). Host errors: num_rows < 0 (GDN_ERR_SHAPE), a missing required
 * pointer or only one of bnd_len / bnd_slot (GDN_ERR_NULL). num_rows == 0
 * returns GDN_OK without a launch.
 */
int32_t gdn_check_slots(int32_t num_rows, const int32_t* src_slot, const int32_t* dst_slot,
                        const int32_t* rec_slot, const int32_t* n_accept,
                        const int32_t* bnd_len, const int32_t* bnd_slot, int32_t* err_flags,
                        void* stream);

/*
 * gdn_native_window -- the baseline being replaced: the same verify
 * arithmetic, but the state after every draft token is written out
 * ([vLLM] Purpose: native spec decode snapshots the full state after every
 * draft position; [TS] Motivation). Bit-identical outputs to gdn_verify.
 *
 * snap: device, [num_rows][HV][T][V][K] in the pool's state dtype (T =
 *   pools->rec_tokens); snap[b][h][t] = state after token t of row b, rounded
 *   to bf16 for bf16 pools. 16-byte aligned. No record is written.
 * Rows: as gdn_verify without record slot and ring base (and its limit on
 * num_rows * HV).
 */
int32_t gdn_native_window(const gdn_pools* pools, int32_t layer, int32_t num_rows,
                          const int32_t* state_slot, const int32_t* tok_start,
                          const int32_t* win_len, const gdn_verify_io* io, void* snap,
                          int32_t* err_flags, void* stream);

/*
 * gdn_native_accept -- the baseline's state copy: for every layer, row b
 * with n = n_accept[b] >= 1 copies snap_layers[l][b][h][n-1] into
 * state[l][dst_slot[b]][h]. snap_layers: host array of num_layers device
 * pointers laid out as in gdn_native_window. One 256-thread workgroup per
 * (layer, row, head): GDN_ERR_SHAPE when there are more than (2^32 - 1) / 256.
 */
int32_t gdn_native_accept(const gdn_pools* pools, void* const* snap_layers,
                          int32_t num_rows, const int32_t* dst_slot,
                          const int32_t* n_accept, int32_t* err_flags, void* stream);

/* Floats per (record slot, value head) block of a correction record:
 * T*(V+K) + T rounded up to 4 (0 for T < 1). */
int64_t gdn_rec_stride(int32_t rec_tokens);

/* Floats per (record slot, value head) block of a record kind (payload:
 * (T*(K+V)*2 + 8*T) bytes rounded up to 16, in floats; per-channel decay:
 * T*(V+2K)); 0 for T < 1 or an unknown kind. */
int64_t gdn_record_stride(int32_t rec_tokens, int32_t record_kind);

const char* gdn_status_string(int32_t status);
int32_t gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_REPLAY_H */
