// gdn_commit.hip -- the all-layer commit (replay of the accepted prefix) and the
// native baseline's accepted-state copy, for gfx950.
//
// Method: vLLM PR "[Spec Decode][Qwen4Exp] RecoverSSM for Qwen GDN and the PLE
// short conv" -- Purpose (after sampling, replay only the accepted tokens and
// write the state once; align mode also writes the block-boundary state),
// Test Result (the replay update is h = fma(correction, key, h * decay), which
// makes the committed state equal to the native per-token state bit for bit),
// Commits items 4 and 6 (one fold per program; final states before boundary
// states, a boundary whose slot is the final slot skipped). tokenspeed PR
// "feat: add Qwen3.5 GDN ReplaySSM", Summary and Implementation (one replay
// launch over all layers; a cooperative block of four warps per 128x128 head).
//
// One launch over (layer, row, value head, part): a head is split over 8
// (fp32) or 4 (bf16) workgroups of four wave64s, 8 KiB of state each, each
// owning a contiguous run of its rows. A thread first loads its share of the
// n records (the workgroup's rows of the corrections, all of the keys, the
// decays), then its 16-byte pieces of the source head -- thread t owns pieces
// t + 256*i, so each load instruction of the workgroup covers 4 KiB of
// contiguous memory. Loads complete in issue order, so the records arrive
// first. They are staged in LDS, and the replay (elementwise, no reductions)
// runs token by token over the thread's pieces: the pieces share their
// columns, so each token's key and decay are read from LDS once, and the
// first token's pass waits for each piece's own load in turn, overlapping the
// transfer of the later pieces. The final state is stored, then in align mode
// the boundary state kept in a second register tile. State loads and stores
// are nontemporal (streamed past the caches: nothing here is reused), and the
// workgroup ids are remapped so that each XCD streams a contiguous range of
// heads. Launches are held to six workgroups per CU through their LDS
// request (fewer bytes in flight per CU stream faster), except align-mode
// launches over more than eight records. Because every thread reads all of
// its source elements before its first store and writes only the elements it
// read, a destination or boundary slot equal to the source slot is safe; the
// pages' read-after-overwrite race between programs cannot occur.
//
// The same launch optionally carries the short conv's state compaction (extra
// workgroups ahead of the replay's, so that their short copies overlap the
// replay's ramp-up rather than its drain) and serves two more record kinds:
// the payload kind, whose replay recomputes each correction from the recorded
// key and value, and the per-key-channel decay kind (a reading of Kimi-K3
// KDA), whose replay is h[v][k] = fma(delta[v], k_hat[k], h[v][k] * alpha[k]).
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

#pragma clang fp contract(off)

namespace gdn {
namespace {

// Ownership of the elements of one head. The head is cut into 16-byte pieces
// (fp32: 4096 pieces of 4 values, piece f = row f/32, columns 4*(f%32)..+3;
// bf16: 2048 pieces of 8 values, piece f = row f/16, columns 8*(f%16)..+7) and
// split over SPLIT workgroups: workgroup `part` owns a contiguous run of
// 128/SPLIT rows, and its thread t owns pieces base + t + 256*i. Each load or
// store instruction of a workgroup therefore covers 4 KiB of contiguous memory.
template <typename StateT, int SPLIT> struct HeadIO;

template <int SPLIT> struct HeadIO<float, SPLIT> {
    static constexpr int kPer = 16 / SPLIT;              // pieces (f32x4) per thread
    __device__ static int piece(int part, int t, int i) { return part * (4096 / SPLIT) + t + kThreads * i; }
    __device__ static void load(const float* head, int part, int t, f32x4 (&h)[kPer]) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) h[i] = ld4_nt(head + 4 * piece(part, t, i));
    }
    __device__ static void store(float* head, int part, int t, const f32x4 (&h)[kPer]) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) st4_nt(head + 4 * piece(part, t, i), h[i]);
    }
    // row of piece i relative to the workgroup's first row: (t / 32) + 8 i
    __device__ static int local_row(int t, int i) { return (t + kThreads * i) >> 5; }
    __device__ static int col0(int t) { return 4 * (t & 31); }
    // a thread owns kOwnRows rows, one per piece, kGroup rows apart; in the
    // permuted correction order drow they are contiguous
    static constexpr int kGroup = kThreads / 32, kOwnRows = kPer;
    __device__ static int drow(int r) { return (r % kGroup) * kOwnRows + r / kGroup; }
};

template <int SPLIT> struct HeadIO<uint16_t, SPLIT> {
    static constexpr int kPieces = 8 / SPLIT;            // 16-byte pieces per thread
    static constexpr int kPer = 2 * kPieces;             // held as f32x4 halves
    __device__ static int piece(int part, int t, int i) { return part * (2048 / SPLIT) + t + kThreads * i; }
    __device__ static void load(const uint16_t* head, int part, int t, f32x4 (&h)[kPer]) {
#pragma unroll
        for (int i = 0; i < kPieces; ++i) {
            const u32x4 x = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(head + 8 * piece(part, t, i)));
            h[2 * i] = f32x4{bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y)};
            h[2 * i + 1] = f32x4{bf16_lo(x.z), bf16_hi(x.z), bf16_lo(x.w), bf16_hi(x.w)};
        }
    }
    __device__ static void store(uint16_t* head, int part, int t, const f32x4 (&h)[kPer]) {
#pragma unroll
        for (int i = 0; i < kPieces; ++i) {
            const f32x4 a = h[2 * i], c = h[2 * i + 1];
            const u32x4 x{pack_bf16(a.x, a.y), pack_bf16(a.z, a.w), pack_bf16(c.x, c.y),
                          pack_bf16(c.z, c.w)};
            __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(head + 8 * piece(part, t, i)));
        }
    }
    // row of piece pair i relative to the workgroup's first row: (t / 16) + 16 i
    __device__ static int local_row(int t, int i) { return (t + kThreads * i) >> 4; }
    __device__ static int col0(int t) { return 8 * (t & 15); }
    static constexpr int kGroup = kThreads / 16, kOwnRows = kPieces;
    __device__ static int drow(int r) { return (r % kGroup) * kOwnRows + r / kGroup; }
};

// Row check shared by the state replay and the conv compaction of one launch:
// a row with bad data is skipped by both parts.
template <bool ALIGN>
__device__ int commit_row_error(const CommitParams& p, int b, int n, int src, int dst, int bl, int bs)
{
    int err = 0;
    if (n < 0 || dst < 0) err |= kRowN;
    if (ALIGN && bl != 0 && (bl < 0 || bl >= n || bs < 0)) err |= kRowBnd;
    if (p.ssm_wgs > 0) {
        const int rs = p.rec_slot[b];
        if (n > p.T) err |= kRowN;
        if (src >= p.num_slots || dst >= p.num_slots) err |= kRowSlot;
        if (ALIGN && bl > 0 && bs >= p.num_slots) err |= kRowBnd;
        if (rs < 0 || rs >= p.num_rec_slots) err |= kRowRec;
    }
    if (p.conv_wgs > 0) {
        const int ts = p.conv.tok_start[b];
        if (src >= p.conv.num_slots || dst >= p.conv.num_slots) err |= kRowSlot;
        if (ALIGN && bl > 0 && bs >= p.conv.num_slots) err |= kRowBnd;
        if (ts < 0 || (int64_t)ts + n > p.conv.num_tokens) err |= kRowWin;
    }
    return err;
}

// Short-conv state compaction of one (layer, row, chunk of 256 16-byte column
// pieces): row i of the final state is row n + i of [source rows 0..Ls-1,
// inputs x_0..x_{n-1}], row i of the boundary state row bnd_len + i. Each
// thread copies one column piece down the rows, in ascending i; it reads row
// n + i (or bnd_len + i > i) before it writes row i, so one state written over
// its own source is shifted in place correctly. Both states must be formed
// from unmodified source rows: when the final state goes into the source slot
// (and the boundary, since it is written at all, into another slot), the
// boundary rows are copied first; otherwise the final rows come first, and a
// boundary written into the source slot then shifts it in place. No
// arithmetic: the bytes are moved as they are.
template <bool ALIGN>
__device__ void conv_compact(const CommitParams& p, int64_t id)
{
    static_assert(kConvPiecesPerWg == kThreads, "one piece per thread");
    const ConvParams& c = p.conv;
    const uint32_t lb = udiv((uint32_t)id, c.div_wpr);
    const int chunk = (int)((uint32_t)id - lb * (uint32_t)c.wgs_per_row);
    const int layer = (int)udiv(lb, p.div_rows);
    const int b = (int)(lb - (uint32_t)layer * (uint32_t)p.num_rows);
    const int n = p.n[b];
    if (n == 0) return;
    const int src = p.src[b];
    if (src < 0) return;
    const int dst = p.dst[b];
    const int ts = c.tok_start[b];
    int bl = 0, bs = -1;
    if constexpr (ALIGN) {
        bl = p.bnd_len[b];
        bs = p.bnd_slot[b];
    }
    const int err = commit_row_error<ALIGN>(p, b, n, src, dst, bl, bs);
    if (err) {
        if (threadIdx.x == 0 && chunk == 0 && layer == 0 && p.err) atomicOr(p.err, err);
        return;
    }
    const int piece = chunk * kThreads + (int)threadIdx.x;
    if (piece >= c.pieces) return;
    const int Ls = c.state_len;
    const int64_t slot_bytes = (int64_t)Ls * c.row_bytes;
    char* pool = static_cast<char*>(c.state[layer]) + 16 * (int64_t)piece;
    const char* srcp = pool + src * slot_bytes;
    const char* xp = static_cast<const char*>(c.x[layer]) + (int64_t)ts * c.x_tok_bytes + 16 * (int64_t)piece;
    auto row = [&](int r) -> u32x4 {
        const char* q = r < Ls ? srcp + r * c.row_bytes : xp + (int64_t)(r - Ls) * c.x_tok_bytes;
        return *reinterpret_cast<const u32x4*>(q);
    };
    char* dstp = pool + dst * slot_bytes;
    auto write_final = [&]() {
        for (int i = 0; i < Ls; ++i) *reinterpret_cast<u32x4*>(dstp + i * c.row_bytes) = row(n + i);
    };
    if constexpr (ALIGN) {
        if (bl > 0 && bs != dst) {
            char* bp = pool + bs * slot_bytes;
            auto write_bnd = [&]() {
                for (int i = 0; i < Ls; ++i) *reinterpret_cast<u32x4*>(bp + i * c.row_bytes) = row(bl + i);
            };
            if (dst == src) {       // the final shift would overwrite rows the boundary reads
                write_bnd();
                write_final();
            } else {
                write_final();
                write_bnd();
            }
            return;
        }
    }
    write_final();
}

template <typename StateT, bool ALIGN, int SPLIT, bool CONV, bool PAY, bool CH>
__global__ void __launch_bounds__(kThreads) commit_kernel(CommitParams p)
{
    // the conv compaction's workgroups come first, their count padded to a
    // multiple of the XCD count so that the replay's ids below keep the
    // hardware's round-robin XCD assignment
    const int64_t conv_off = CONV ? (p.conv_wgs + kNumXcd - 1) / kNumXcd * kNumXcd : 0;
    if constexpr (CONV) {
        if ((int64_t)blockIdx.x < conv_off) {
            if ((int64_t)blockIdx.x < p.conv_wgs) conv_compact<ALIGN>(p, (int64_t)blockIdx.x);
            return;
        }
    }
    typedef HeadIO<StateT, SPLIT> IO;
    constexpr int kRows = kDim / SPLIT;   // rows of the head this workgroup owns
    extern __shared__ float lds[];
    const int T = p.T;
    float* d_l = lds;                 // [n][kRows] corrections (payload: values) of the owned rows
    float* k_l = lds + T * kDim;      // [n][128] normalised keys
    float* g_l = lds + 2 * T * kDim;  // [n] decays (payload: then [n] write strengths;
                                      // per-channel records: [n][128] decays)

    // logical id: (layer, row, value head, part), XCD-contiguous
    const uint32_t wr = blockIdx.x - (uint32_t)conv_off;
    const uint32_t wg = kCommitXcdRemap ? xcd_contiguous_id(wr, (uint32_t)p.ssm_wgs) : wr;
    const int part = (int)(wg % SPLIT);
    const uint32_t head_id = wg / SPLIT;
    const uint32_t lb = udiv(head_id, p.div_hv);
    const int hv = (int)(head_id - lb * (uint32_t)p.hv);
    const int layer = (int)udiv(lb, p.div_rows);
    const int b = (int)(lb - (uint32_t)layer * (uint32_t)p.num_rows);

    // ---- row decode ----
    const int n = p.n[b];
    if (n == 0) return;
    const int src = p.src[b];
    if (src < 0) return;
    const int dst = p.dst[b];
    const int rs = p.rec_slot[b];
    int bl = 0, bs = -1;
    if constexpr (ALIGN) {
        bl = p.bnd_len[b];
        bs = p.bnd_slot[b];
    }
    const int err = commit_row_error<ALIGN>(p, b, n, src, dst, bl, bs);
    if (err) {
        if (threadIdx.x == 0 && hv == 0 && layer == 0 && part == 0 && p.err) atomicOr(p.err, err);
        return;
    }
    const bool write_bnd = ALIGN && bl > 0 && bs != dst;

    const int t = threadIdx.x;
    StateT* pool = static_cast<StateT*>(p.state[layer]);
    const int64_t slot_elems = (int64_t)p.hv * kHeadElems;
    const int64_t head_off = (int64_t)hv * kHeadElems;
    const float* recb = p.rec[layer] + ((int64_t)rs * p.hv + hv) * p.rec_stride;
    constexpr int kRow4 = kRows / 4;
    const int c0 = IO::col0(t);
    // Records: this thread's share of the n records is loaded before the tile,
    // so it arrives first (loads complete in issue order). Correction records:
    // the owned rows of the corrections, all of the keys, the decays. Payload
    // records: one 16-byte piece of a raw key, the owned rows of the raw values,
    // a decay and a write strength.
    constexpr int kDChunks = (kMaxRecTokens * kRow4 + kThreads - 1) / kThreads;
    constexpr int kKChunks = (kMaxRecTokens * (kDim / 4) + kThreads - 1) / kThreads;
    f32x4 rd[kDChunks], rk[kKChunks], ra[CH ? kKChunks : 1];
    float rg = 0.f, rb = 0.f;
    u32x4 pk = {0u, 0u, 0u, 0u};
    u32x2 pv[kDChunks];
    const uint16_t* kb = reinterpret_cast<const uint16_t*>(recb);
    const uint16_t* vb = kb + (int64_t)T * kDim;
    if constexpr (PAY) {
        static_assert(kMaxRecTokens * kDim / 8 <= kThreads, "one key piece per thread");
        if ((t >> 4) < n) pk = *reinterpret_cast<const u32x4*>(kb + (t >> 4) * kDim + 8 * (t & 15));
#pragma unroll
        for (int q = 0; q < kDChunks; ++q) {
            const int i = t + q * kThreads;
            if (i < n * kRow4) {
                const int tt = i / kRow4;
                pv[q] = *reinterpret_cast<const u32x2*>(vb + tt * kDim + part * kRows + 4 * (i - tt * kRow4));
            }
        }
        if (t < n) {
            rg = recb[(int64_t)T * kDim + t];
            rb = recb[(int64_t)T * (kDim + 1) + t];
        }
    } else {
#pragma unroll
        for (int q = 0; q < kDChunks; ++q) {
            const int i = t + q * kThreads;
            if (i < n * kRow4) {
                const int tt = i / kRow4;
                rd[q] = ld4(recb + tt * kDim + part * kRows + 4 * (i - tt * kRow4));
            }
        }
#pragma unroll
        for (int q = 0; q < kKChunks; ++q) {
            const int i = t + q * kThreads;
            if (i < n * (kDim / 4)) rk[q] = ld4(recb + (int64_t)T * kDim + 4 * i);
        }
        if constexpr (CH) {   // per-channel decays, laid out like the keys
#pragma unroll
            for (int q = 0; q < kKChunks; ++q) {
                const int i = t + q * kThreads;
                if (i < n * (kDim / 4)) ra[q] = ld4(recb + 2 * (int64_t)T * kDim + 4 * i);
            }
        }
        if (t < n) rg = recb[2 * (int64_t)T * kDim + t];
    }
    f32x4 h[IO::kPer];
    IO::load(pool + src * slot_elems + head_off, part, t, h);

    if constexpr (PAY) {
        // ---- payload records into LDS: keys normalised with the same helper
        // as verify (so the same bits), the owned rows of the values widened ----
        float* b_l = g_l + T;             // [n] write strengths
        if ((t >> 4) < n) {               // uniform over each 16-lane row of the reduction
            float x[8] = {bf16_lo(pk.x), bf16_hi(pk.x), bf16_lo(pk.y), bf16_hi(pk.y),
                          bf16_lo(pk.z), bf16_hi(pk.z), bf16_lo(pk.w), bf16_hi(pk.w)};
            l2norm_row16(x);
            float* kp = k_l + (t >> 4) * kDim + 8 * (t & 15);
            st4(kp, f32x4{x[0], x[1], x[2], x[3]});
            st4(kp + 4, f32x4{x[4], x[5], x[6], x[7]});
        }
#pragma unroll
        for (int q = 0; q < kDChunks; ++q) {
            const int i = t + q * kThreads;
            if (i < n * kRow4)
                st4(d_l + 4 * i, f32x4{bf16_lo(pv[q].x), bf16_hi(pv[q].x), bf16_lo(pv[q].y), bf16_hi(pv[q].y)});
        }
        if (t < n) {
            g_l[t] = rg;
            b_l[t] = rb;
        }
        __syncthreads();

        // ---- replay piece by piece with recomputed corrections: h' = g h,
        // u = h' k_hat (a reduction over the lanes holding the piece's row: 32
        // for fp32, 16 for bf16), delta = beta (v - u), h = fma(delta, k_hat, h').
        // A row lies within one piece index, so each piece waits only for its
        // own load. ----
        f32x4 hb[ALIGN ? IO::kPer : 1];
        if constexpr (sizeof(StateT) == 4) {
#pragma unroll
            for (int i = 0; i < IO::kPer; ++i) {
                const int row = IO::local_row(t, i);
                for (int tt = 0; tt < n; ++tt) {
                    const float g = g_l[tt], be = b_l[tt];
                    const f32x4 kh = ld4(k_l + tt * kDim + c0);
                    f32x4 hp;
                    float acc = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        hp[e] = h[i][e] * g;
                        acc = __builtin_fmaf(hp[e], kh[e], acc);
                    }
                    const float d = be * (d_l[tt * kRows + row] - sum32(acc));
#pragma unroll
                    for (int e = 0; e < 4; ++e) h[i][e] = __builtin_fmaf(d, kh[e], hp[e]);
                    if constexpr (ALIGN) {
                        if (tt + 1 == bl) hb[i] = h[i];
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < IO::kPer / 2; ++i) {
                const int row = IO::local_row(t, i);
                for (int tt = 0; tt < n; ++tt) {
                    const float g = g_l[tt], be = b_l[tt];
                    const f32x4 kh0 = ld4(k_l + tt * kDim + c0);
                    const f32x4 kh1 = ld4(k_l + tt * kDim + c0 + 4);
                    f32x4 hp0, hp1;
                    float acc = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        hp0[e] = h[2 * i][e] * g;
                        acc = __builtin_fmaf(hp0[e], kh0[e], acc);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        hp1[e] = h[2 * i + 1][e] * g;
                        acc = __builtin_fmaf(hp1[e], kh1[e], acc);
                    }
                    const float d = be * (d_l[tt * kRows + row] - sum16(acc));
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        h[2 * i][e] = __builtin_fmaf(d, kh0[e], hp0[e]);
                        h[2 * i + 1][e] = __builtin_fmaf(d, kh1[e], hp1[e]);
                    }
                    if constexpr (ALIGN) {
                        if (tt + 1 == bl) {
                            hb[2 * i] = h[2 * i];
                            hb[2 * i + 1] = h[2 * i + 1];
                        }
                    }
                }
            }
        }
        // ---- final state first, then the boundary state ----
        IO::store(pool + dst * slot_elems + head_off, part, t, h);
        if constexpr (ALIGN) {
            if (write_bnd) IO::store(pool + bs * slot_elems + head_off, part, t, hb);
        }
    } else {
    // ---- the n records into LDS. The corrections of token tt are kept
    // row-permuted: row r of the workgroup sits at tt*kRows + IO::drow(r), so
    // that the rows one thread owns come in one or two vector reads a token ----
#pragma unroll
    for (int q = 0; q < kDChunks; ++q) {
        const int i = t + q * kThreads;
        if (i < n * kRow4) {
            const int tt = i / kRow4;
            const int r = 4 * (i - tt * kRow4);
            float* dp = d_l + tt * kRows;
#pragma unroll
            for (int e = 0; e < 4; ++e) dp[IO::drow(r + e)] = rd[q][e];
        }
    }
#pragma unroll
    for (int q = 0; q < kKChunks; ++q) {
        const int i = t + q * kThreads;
        if (i < n * (kDim / 4)) st4(k_l + 4 * i, rk[q]);
    }
    if constexpr (CH) {
#pragma unroll
        for (int q = 0; q < kKChunks; ++q) {
            const int i = t + q * kThreads;
            if (i < n * (kDim / 4)) st4(g_l + 4 * i, ra[q]);
        }
    } else {
        if (t < n) g_l[t] = rg;
    }
    __syncthreads();

    // ---- replay, h = fma(delta_t[row], k_hat_t[col], h * g_t) for t < n,
    // token by token over the thread's pieces ----
    f32x4 hb[ALIGN ? IO::kPer : 1];
    constexpr int kOwn = IO::kOwnRows;
    static_assert(IO::kGroup * kOwn == kRows && kOwn % 2 == 0, "permuted correction rows");
    const float* d_own = d_l + IO::drow(IO::local_row(t, 0));
    for (int tt = 0; tt < n; ++tt) {
        float d[kOwn];
        if constexpr (kOwn % 4 == 0) {
#pragma unroll
            for (int j = 0; j < kOwn; j += 4) {
                const f32x4 x = ld4(d_own + tt * kRows + j);
#pragma unroll
                for (int e = 0; e < 4; ++e) d[j + e] = x[e];
            }
        } else {
#pragma unroll
            for (int j = 0; j < kOwn; j += 2) {
                const f32x2 x = *reinterpret_cast<const f32x2*>(d_own + tt * kRows + j);
                d[j] = x.x;
                d[j + 1] = x.y;
            }
        }
        if constexpr (sizeof(StateT) == 4) {
            const f32x4 kh = ld4(k_l + tt * kDim + c0);
            if constexpr (CH) {          // per-channel decay, column by column
                const f32x4 al = ld4(g_l + tt * kDim + c0);
#pragma unroll
                for (int i = 0; i < IO::kPer; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) h[i][e] = __builtin_fmaf(d[i], kh[e], h[i][e] * al[e]);
            } else {
                const float g = g_l[tt];
#pragma unroll
                for (int i = 0; i < IO::kPer; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) h[i][e] = __builtin_fmaf(d[i], kh[e], h[i][e] * g);
            }
        } else {
            const f32x4 kh0 = ld4(k_l + tt * kDim + c0);
            const f32x4 kh1 = ld4(k_l + tt * kDim + c0 + 4);
            if constexpr (CH) {
                const f32x4 al0 = ld4(g_l + tt * kDim + c0);
                const f32x4 al1 = ld4(g_l + tt * kDim + c0 + 4);
#pragma unroll
                for (int i = 0; i < IO::kPer / 2; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        h[2 * i][e] = __builtin_fmaf(d[i], kh0[e], h[2 * i][e] * al0[e]);
                        h[2 * i + 1][e] = __builtin_fmaf(d[i], kh1[e], h[2 * i + 1][e] * al1[e]);
                    }
            } else {
                const float g = g_l[tt];
#pragma unroll
                for (int i = 0; i < IO::kPer / 2; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        h[2 * i][e] = __builtin_fmaf(d[i], kh0[e], h[2 * i][e] * g);
                        h[2 * i + 1][e] = __builtin_fmaf(d[i], kh1[e], h[2 * i + 1][e] * g);
                    }
            }
        }
        if constexpr (ALIGN) {
            if (tt + 1 == bl) {
#pragma unroll
                for (int i = 0; i < IO::kPer; ++i) hb[i] = h[i];
            }
        }
    }

    // ---- final state first, then the boundary state ----
    IO::store(pool + dst * slot_elems + head_off, part, t, h);
    if constexpr (ALIGN) {
        if (write_bnd) IO::store(pool + bs * slot_elems + head_off, part, t, hb);
    }
    }
}

// Native baseline: copy the snapshot of the last accepted token into the slot.
template <typename StateT>
__global__ void __launch_bounds__(kThreads) accept_kernel(AcceptParams p)
{
    const uint32_t wg = blockIdx.x;
    const uint32_t lb = udiv(wg, p.div_hv);
    const int hv = (int)(wg - lb * (uint32_t)p.hv);
    const int layer = (int)udiv(lb, p.div_rows);
    const int b = (int)(lb - (uint32_t)layer * (uint32_t)p.num_rows);
    const int n = p.n[b];
    if (n == 0) return;
    const int dst = p.dst[b];
    int err = 0;
    if (n < 0 || n > p.T || dst < 0) err |= kRowN;
    if (dst >= p.num_slots) err |= kRowSlot;
    if (err) {
        if (threadIdx.x == 0 && hv == 0 && layer == 0 && p.err) atomicOr(p.err, err);
        return;
    }
    const StateT* sn = static_cast<const StateT*>(p.snap[layer]) +
                       (((int64_t)b * p.hv + hv) * p.T + (n - 1)) * kHeadElems;
    StateT* out = static_cast<StateT*>(p.state[layer]) + ((int64_t)dst * p.hv + hv) * kHeadElems;
    constexpr int kPer = (int)(kHeadElems * sizeof(StateT) / 16 / kThreads);
    const f32x4* s4 = reinterpret_cast<const f32x4*>(sn);
    f32x4* o4 = reinterpret_cast<f32x4*>(out);
    f32x4 x[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) x[i] = s4[threadIdx.x + kThreads * i];
#pragma unroll
    for (int i = 0; i < kPer; ++i) __builtin_nontemporal_store(x[i], o4 + threadIdx.x + kThreads * i);
}

// LDS requested per workgroup. A launch asks for at least kLdsFloor bytes,
// which holds it to six workgroups per CU (of 160 KiB) where the waves alone
// would allow eight: 48 KiB of state in flight per CU instead of 64, which HBM
// streams faster. The exception is an align-mode launch with more than
// kAlignFloorRecTokens records: with its long record staging and the second
// (boundary) store it streams as well or better at full occupancy.
constexpr int kAlignFloorRecTokens = 8;
constexpr size_t kLdsFloor = 24 * 1024;
size_t commit_lds_request(int T, bool channel, bool align)
{
    const size_t need = commit_lds_bytes(T, channel);
    const bool capped = !align || T <= kAlignFloorRecTokens;
    return capped && need < kLdsFloor ? kLdsFloor : need;
}

template <typename StateT, bool ALIGN, int SPLIT>
hipError_t launch_c(const CommitParams& p, hipStream_t s)
{
    static_assert(kThreads == kCommitThreads, "launch limit counted for 256-thread workgroups");
    const bool conv = p.conv_wgs > 0;
    const void* fn =
        p.payload   ? (conv ? reinterpret_cast<const void*>(&commit_kernel<StateT, ALIGN, SPLIT, true, true, false>)
                            : reinterpret_cast<const void*>(&commit_kernel<StateT, ALIGN, SPLIT, false, true, false>))
        : p.channel ? (conv ? reinterpret_cast<const void*>(&commit_kernel<StateT, ALIGN, SPLIT, true, false, true>)
                            : reinterpret_cast<const void*>(&commit_kernel<StateT, ALIGN, SPLIT, false, false, true>))
                    : (conv ? reinterpret_cast<const void*>(&commit_kernel<StateT, ALIGN, SPLIT, true, false, false>)
                            : reinterpret_cast<const void*>(&commit_kernel<StateT, ALIGN, SPLIT, false, false, false>));
    // workgroups of one layer: the state replay's and the conv compaction's
    const int64_t ssm_layer = p.hv > 0 ? (int64_t)p.num_rows * p.hv * SPLIT : 0;
    const int64_t conv_layer = conv ? (int64_t)p.num_rows * p.conv.wgs_per_row : 0;
    // layers per launch: all of them unless the grid would pass the
    // dispatch limit (the host entry point has checked that one layer fits)
    if (ssm_layer + conv_layer == 0) return hipSuccess;
    const int64_t per = (kMaxLaunchWgs - kNumXcd) / (ssm_layer + conv_layer);
    if (per < 1) return hipErrorInvalidConfiguration;
    const int step = per >= p.num_layers ? p.num_layers : (int)per;
    for (int l0 = 0; l0 < p.num_layers; l0 += step) {
        CommitParams args = p;
        const int nl = p.num_layers - l0 < step ? p.num_layers - l0 : step;
        for (int l = 0; l < nl; ++l) {
            args.state[l] = p.state[l0 + l];
            args.rec[l] = p.rec[l0 + l];
            args.conv.state[l] = p.conv.state[l0 + l];
            args.conv.x[l] = p.conv.x[l0 + l];
        }
        args.num_layers = nl;
        args.ssm_wgs = ssm_layer * nl;
        args.conv_wgs = conv_layer * nl;
        const int64_t conv_off = conv ? (args.conv_wgs + kNumXcd - 1) / kNumXcd * kNumXcd : 0;
        const uint64_t grid = (uint64_t)(args.ssm_wgs + conv_off);
        void* kargs[] = {&args};
        const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kThreads), kargs,
                                             commit_lds_request(p.T, p.channel, ALIGN), s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Workgroups per head: 8 KiB of state per workgroup, 8 per head for fp32 pools
// and 4 for bf16 pools, whatever the record capacity.
template <bool ALIGN>
hipError_t launch_c_split(const CommitParams& p, bool bf16_state, hipStream_t s)
{
    if (bf16_state) {
        static_assert(kCommitSplitBf16 == 4, "bf16 split");
        return launch_c<uint16_t, ALIGN, kCommitSplitBf16>(p, s);
    }
    static_assert(kCommitSplitF32 == 8, "fp32 split");
    return launch_c<float, ALIGN, kCommitSplitF32>(p, s);
}

template <typename StateT>
hipError_t launch_a(const AcceptParams& p, hipStream_t s)
{
    AcceptParams args = p;
    void* kargs[] = {&args};
    const uint64_t grid = (uint64_t)p.num_layers * p.num_rows * p.hv;
    return hipLaunchKernel(reinterpret_cast<const void*>(&accept_kernel<StateT>),
                           dim3((unsigned)grid), dim3(kThreads), kargs, 0, s);
}

}  // namespace

hipError_t launch_commit(const CommitParams& p, bool bf16_state, bool align, hipStream_t s)
{
    return align ? launch_c_split<true>(p, bf16_state, s) : launch_c_split<false>(p, bf16_state, s);
}

hipError_t launch_native_accept(const AcceptParams& p, bool bf16_state, hipStream_t s)
{
    return bf16_state ? launch_a<uint16_t>(p, s) : launch_a<float>(p, s);
}

}  // namespace gdn
