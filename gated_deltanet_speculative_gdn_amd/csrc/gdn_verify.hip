// gdn_verify.hip -- verify from a read-only checkpoint, and the native
// snapshot-every-token baseline, for gfx950.
//
// Method: vLLM PR "[Spec Decode][Qwen4Exp] RecoverSSM for Qwen GDN and the PLE
// short conv", Purpose (verify runs the draft window from the checkpoint,
// writes the per-token outputs and an fp32 record of correction, normalised key
// and gate, never the state) and Test Result (the record holds the decay that
// was multiplied in; the commit's forward replay of it equals the native
// per-token state bit for bit); the rule itself is the gated delta rule of
// "Gated Delta Networks" (Yang, Kautz, Hatamizadeh, ICLR 2025). Ring mode
// (records of earlier single-token steps applied before the window) follows the
// 16-token replay buffer of lmdeploy PR #5028 (Performance test settings).
//
// Verify never writes the state, so it never forms S_t. With the positions
// 0..P-1 of a row (0..j0-1: pending ring records, j0..P-1: the window), the
// decay products G(a, b) = g_a * ... * g_{b-1} and the checkpoint S0, the rule
// S_{p+1} = g_p S_p + delta_p k_p^T unrolls to
//   u_p = G(0,p+1) (S0 k_p) + sum_{j<p}  G(j+1,p+1) (k_j . k_p) delta_j
//   o_p = G(0,p+1) (S0 q_p) + sum_{j<=p} G(j+1,p+1) (k_j . q_p) delta_j
//   delta_p = beta_p (v_p - u_p)
// (k, q normalised; q scaled). The only work proportional to the 128x128 head
// is the contraction of S0 with the 2w window vectors: 2w fmas per state
// element instead of the per-token rule's 4w operations, and ring records cost
// a scalar term each instead of a pass over the head. The 2w-column product is
// a dense contraction and its fmas are what separate this kernel from its
// memory floor, but matrix-core versions measured slower (fp32 16x16x4 with half
// of the columns idle at w = 4; 4x4x1 with none idle): the products then make a
// round trip through LDS to a per-row recurrence, which costs more than the
// vector fmas it saves. On bf16 pools a 16x16x32 bf16 version (the window
// vectors split exactly into three bf16 parts) halves the vector instructions,
// but the matrix layout wants sixteen rows across neighbouring lanes where the
// coalesced loads put one row: moving the tile between the two layouts with
// lane permutes costs as much LDS time as the fmas save, and loading it in the
// matrix layout halves the row segments each load covers. So the contraction
// stays on the vector ALU, fused with the recurrence in registers.
//
// One workgroup per (row, value head, chunk of NT/8*R head rows): eight wave64s
// covering the whole head for windows of up to 4 positions, four wave64s per
// half head for longer ones;
// workgroup ids are remapped so that each XCD streams a contiguous stretch of
// the pool. Thread t holds head rows row0 + R*(t/8) + r and 16 of their
// columns, 4*(t%8) + 32*c + e (c, e = 0..3) on fp32 pools and 8*(t%8) + 64*m + e
// (m = 0..1, e = 0..7) on bf16 pools: either way each 16-byte load of eight
// neighbouring lanes covers a whole 128-byte row segment, and a length-128
// reduction is 16
// fmas in the lane plus three DPP steps over the eight lanes of a row group,
// arranged so that lanes 0-3 end with the even rows' sums and lanes 4-7 with
// the odd rows' (the per-row recurrence then runs in four lanes per row, not
// eight). The window's vectors and the per-item scalar coefficients are staged
// in LDS once.
//
// Options carried in the parameters: gates formed here from raw projections
// (A_log, dt_bias), outputs rounded to bf16, and payload records (the raw key
// and value with the gates) in place of the corrections. A template flag (CH)
// takes one decay per key channel (a reading of Kimi-K3 KDA, which the vLLM
// PR's Purpose names as a user of the same protocol): the decay products
// become elementwise, G(a, b) = alpha_a * ... * alpha_{b-1} per channel, so
// S0 is contracted with G(0,p+1) * k_p and G(0,p+1) * q_p and each
// coefficient is the dot product of k_j * G(j+1,p+1) with k_p or q_p; the
// record keeps alpha[K] in place of the gate.
//
// The native baseline is the same template with SNAP = true: the same
// corrections and outputs, bit for bit, then the states S_1..S_w materialised
// with the commit's update h = fma(delta, k, h * g) and written out -- so the
// commit's replay of verify's records reproduces the baseline's states exactly.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

#pragma clang fp contract(off)

namespace gdn {
namespace {

// ---- register tile of R rows: h[r][c] = row row0 + R*grp + r, the four
// columns tcol<StateT>(lane8, c) .. +3. Each load instruction of an 8-lane
// group reads 128 contiguous bytes of a row: fp32 pools 16 bytes a lane, chunk
// c at column 32c + 4 lane8; bf16 pools 16 bytes (eight values) a lane, chunk
// pair (2m, 2m+1) at column 64m + 8 lane8. (Eight-byte bf16 pieces in the fp32
// column order read 64-byte segments and made the bf16 verify about 5%
// slower.) The lanes' partial sums therefore cover other columns on bf16
// pools than on fp32 pools: the two paths agree to rounding, not bit for bit.
template <typename StateT> __device__ __forceinline__ int tcol(int lane8, int c);
template <> __device__ __forceinline__ int tcol<float>(int lane8, int c) { return 4 * lane8 + 32 * c; }
template <> __device__ __forceinline__ int tcol<uint16_t>(int lane8, int c)
{
    return 8 * lane8 + 64 * (c >> 1) + 4 * (c & 1);
}

template <typename StateT, int R> struct TileIO;

template <int R> struct TileIO<float, R> {
    __device__ static void load(const float* head, int row0, int grp, int lane8, f32x4 (&h)[R][4]) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                h[r][c] = ld4_nt(head + (row0 + R * grp + r) * kDim + tcol<float>(lane8, c));
    }
    __device__ static void store(float* head, int row0, int grp, int lane8, const f32x4 (&h)[R][4]) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                st4_nt(head + (row0 + R * grp + r) * kDim + tcol<float>(lane8, c), h[r][c]);
    }
};

// bf16 pool: one 16-byte piece (eight values) per chunk pair, widened exactly.
template <int R> struct TileIO<uint16_t, R> {
    __device__ static void load(const uint16_t* head, int row0, int grp, int lane8,
                                f32x4 (&h)[R][4]) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                    head + (row0 + R * grp + r) * kDim + tcol<uint16_t>(lane8, 2 * m)));
                h[r][2 * m] = f32x4{bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y)};
                h[r][2 * m + 1] = f32x4{bf16_lo(x.z), bf16_hi(x.z), bf16_lo(x.w), bf16_hi(x.w)};
            }
    }
    __device__ static void store(uint16_t* head, int row0, int grp, int lane8,
                                 const f32x4 (&h)[R][4]) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const f32x4 v = h[r][2 * m], u = h[r][2 * m + 1];
                __builtin_nontemporal_store(
                    u32x4{pack_bf16(v.x, v.y), pack_bf16(v.z, v.w), pack_bf16(u.x, u.y),
                          pack_bf16(u.z, u.w)},
                    reinterpret_cast<u32x4*>(head + (row0 + R * grp + r) * kDim +
                                             tcol<uint16_t>(lane8, 2 * m)));
            }
    }
};

// Row-group dot product of the tile with one staged 128-vector, the rows'
// sums split over the group: 16 fmas per row in each lane, then for each pair
// of rows (2m, 2m+1) one exchange between lane i and lane 7-i of the group, in
// which lanes 0-3 keep row 2m's partial sums and lanes 4-7 row 2m+1's, and two
// exchanges inside each half. out[m] is row 2m's sum in lanes 0-3 and row
// 2m+1's in lanes 4-7 (hi), identical in the four lanes of a half: five
// instructions a pair where a sum in all eight lanes would take six, and the
// per-row arithmetic that follows is done by half as many lanes per row.
template <typename StateT, int R>
__device__ __forceinline__ void tile_dot_split(const f32x4 (&h)[R][4], const float* x, int lane8, bool hi,
                                               float (&out)[R / 2])
{
    f32x4 xv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) xv[c] = ld4(x + tcol<StateT>(lane8, c));
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        acc[r] = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[r] = __builtin_fmaf(h[r][c][e], xv[c][e], acc[r]);
    }
#pragma unroll
    for (int m = 0; m < R / 2; ++m) {
        const float keep = hi ? acc[2 * m + 1] : acc[2 * m];
        const float send = hi ? acc[2 * m] : acc[2 * m + 1];
        float s = keep + dpp<kDppRowHalfMirror>(send);
        s = s + dpp<kDppQuadXor1>(s);
        out[m] = s + dpp<kDppQuadXor2>(s);
    }
}

// LDS layout of one workgroup (floats), TT = compile-time window capacity
// (>= the record capacity T), so every LDS offset is an immediate; RW = the
// head rows the workgroup owns (row0 .. row0+RW-1):
//   khat [TT][128]  normalised keys of every position (ring records and window)
//   qt   [TT][128]  window positions: normalised, scaled queries
//   vd   [TT][RW]   ring positions: recorded corrections; window positions: values
//   dw   [TT][RW]   window positions: the corrections computed here
//   ob   [TT][RW]   window positions: the outputs (written out coalesced at the end)
//   g [TT], be [TT], g0 [TT] = G(0, p+1)
//   ca [TT][TT] = G(j+1, p+1) (k_j . k_p), j < p;  cb [TT][TT] = G(j+1, p+1) (k_j . q_p), j <= p
// Only the keys and queries are needed whole (the dot products); keeping the
// row-indexed fields to the owned rows lets more workgroups share a CU at long
// record capacities.
// With one decay per key channel (CH) more [TT][128] arrays follow:
//   al  the decays of every position;  kx, qx  the window's keys and queries
//   scaled channel by channel by the decay products G(0, p+1), the vectors the
//   checkpoint is contracted with (the scalar G(0, p+1) of the scalar-decay
//   rule is then 1). Only the native baseline (SNAP) keeps kx, qx apart: it
//   still needs the keys themselves afterwards; verify scales khat and qt in
//   place once the coefficients are formed.
template <int TT, int RW, bool CH = false, bool SNAP = false> struct Lds {
    static constexpr size_t kFloats = 2 * TT * kDim + 3 * TT * RW + 3 * TT + 2 * TT * TT +
                                      (CH ? (SNAP ? 3 : 1) * TT * kDim : 0);
    float *khat, *qt, *vd, *dw, *ob, *g, *be, *g0, *ca, *cb, *al, *kx, *qx;
    __device__ explicit Lds(float* base)
        : khat(base), qt(base + TT * kDim), vd(base + 2 * TT * kDim), dw(vd + TT * RW),
          ob(dw + TT * RW), g(ob + TT * RW), be(g + TT), g0(be + TT), ca(g0 + TT), cb(ca + TT * TT),
          al(cb + TT * TT), kx(al + TT * kDim), qx(kx + TT * kDim) {}
};

// NT threads per workgroup, R rows of the head per thread: a workgroup covers
// NT/8 * R rows, so a head is split over kChunks workgroups. Each stages the
// whole window (the norms and dot products need all 128 columns); the
// head-level record fields (key, gate or per-channel decays) are written by
// the first chunk.
template <typename StateT, bool SNAP, int R, int NT, int TT, bool CH>
__global__ void __launch_bounds__(NT) verify_kernel(VerifyParams p)
{
    static_assert(R == 2 || R == 4, "rows per thread: pairs of rows");
    constexpr int kRowsPerWg = NT / 8 * R;
    static_assert(kDim % kRowsPerWg == 0, "workgroup rows divide the head");
    constexpr int kChunks = kDim / kRowsPerWg;
    extern __shared__ float lds_raw[];
    const int T = p.T;   // record capacity (record addressing); T <= TT
    const Lds<TT, kRowsPerWg, CH, SNAP> L(lds_raw);

    const uint32_t item = xcd_contiguous_id(blockIdx.x, gridDim.x);
    const int chunk = (int)(item % kChunks);
    const uint32_t bh = item / kChunks;
    const int b = (int)udiv(bh, p.div_hv);
    const int hv = (int)(bh - (uint32_t)b * (uint32_t)p.hv);
    const int row0 = chunk * kRowsPerWg;
    const bool lead = chunk == 0;

    // ---- row decode: a null slot or an empty window is padding ----
    // (all of the row's metadata is requested before the first wait: one round trip)
    const int slot = ld_uniform(p.state_slot, b);
    const int w = ld_uniform(p.win_len, b);
    const int ts = ld_uniform(p.tok_start, b);
    int j0 = 0, rs = 0;
    if constexpr (!SNAP) {
        j0 = p.rec_base ? ld_uniform(p.rec_base, b) : 0;
        rs = ld_uniform(p.rec_slot, b);
    }
    // consume every value here, so the compiler does not sink the later loads
    // past the padding test into further round trips
    __asm__ volatile("" ::"s"(ts), "s"(j0), "s"(rs));
    if (slot < 0 || w == 0) return;
    int err = 0;
    if (slot >= p.num_slots) err |= kRowSlot;
    if (w < 0 || j0 < 0 || (int64_t)j0 + w > T || ts < 0 || (int64_t)ts + w > p.num_tokens)
        err |= kRowWin;
    if (!SNAP && (rs < 0 || rs >= p.num_rec_slots)) err |= kRowRec;
    if (err) {
        if (threadIdx.x == 0 && p.err) atomicOr(p.err, err);
        return;
    }
    const int P = j0 + w;

    const int tid = threadIdx.x;
    const int lane8 = tid & 7;
    const int grp = tid >> 3;
    const int lane16 = tid & 15;

    // ---- issue the window's loads first, then the checkpoint tile: loads
    // complete in issue order, so the staging below waits only for the small
    // window data and overlaps the tile's transfer ----
    const int hk = hv / p.group;
    // uniform base pointers of the window's first token; a lane's job picks one
    const uint16_t* q_base = p.q + (int64_t)ts * p.q_ts + (int64_t)hk * p.q_hs;
    const uint16_t* k_base = p.k + (int64_t)ts * p.k_ts + (int64_t)hk * p.k_hs;
    const uint16_t* v_base = p.v + (int64_t)ts * p.v_ts + (int64_t)hv * p.v_hs;
    auto job_src = [&](int jb) -> const uint16_t* {
        const int t = jb / 3;
        const int kind = jb - 3 * t;
        const uint16_t* cq = q_base + t * p.q_ts;     // select among addresses, not among
        const uint16_t* ck = k_base + t * p.k_ts;     // argument fields (which would be a
        const uint16_t* cv = v_base + t * p.v_ts;     // per-lane load of the argument block)
        return kind == 0 ? cq : kind == 1 ? ck : cv;
    };
    const int jb0 = tid >> 4;                       // this lane's first (q, k, v) job
    u32x4 raw0 = {0u, 0u, 0u, 0u};
    if (jb0 < 3 * w) raw0 = *reinterpret_cast<const u32x4*>(job_src(jb0) + 8 * lane16);
    // gate inputs of token min(tid, w-1): unconditional, so no use of them is
    // hoisted above the tile loads below
    const int64_t gtok = (int64_t)ts + (tid < w ? tid : w - 1);
    float a_in = 0.f;
    if constexpr (!CH) a_in = p.a_log[gtok * p.g_ts + hv];
    const float b_in = p.beta[gtok * p.g_ts + hv];
    // per-channel log-decays of the window's tokens (CH): 32 16-byte pieces a token
    constexpr int kAChunks = CH ? (TT * (kDim / 4) + NT - 1) / NT : 1;
    f32x4 win_a[kAChunks];
    if constexpr (CH) {
        const float* a_base = p.a_log + (int64_t)ts * p.a_ts + (int64_t)hv * kDim;
#pragma unroll
        for (int q = 0; q < kAChunks; ++q) {
            const int i = tid + q * NT;
            if (i < w * (kDim / 4)) {
                const int t = i / (kDim / 4);
                win_a[q] = ld4(a_base + t * p.a_ts + 4 * (i - t * (kDim / 4)));
            }
        }
    }
    // per-head gate parameters (raw gates); otherwise a harmless in-bounds read
    const float alog_in = (p.raw_gates ? p.A_log : p.a_log)[hv];
    const float dtb_in = (p.raw_gates ? p.dt_bias : p.beta)[hv];
    float* recb = nullptr;
    // pending ring records (positions 0 .. j0-1): the corrections of the owned
    // rows (all this workgroup uses) and all of the keys
    constexpr int kRowQ = kRowsPerWg / 4;
    constexpr int kRingD = (kMaxRecTokens * kRowQ + NT - 1) / NT;
    constexpr int kRingK = (kMaxRecTokens * (kDim / 4) + NT - 1) / NT;
    f32x4 ring_d[kRingD], ring_k[kRingK], ring_a[CH ? kRingK : 1];
    float ring_g = 0.f;
    if constexpr (!SNAP) {
        recb = p.rec + ((int64_t)rs * p.hv + hv) * p.rec_stride;
#pragma unroll
        for (int q = 0; q < kRingD; ++q) {
            const int i = tid + q * NT;
            if (i < j0 * kRowQ) {
                const int t = i / kRowQ;
                ring_d[q] = ld4(recb + t * kDim + row0 + 4 * (i - t * kRowQ));
            }
        }
#pragma unroll
        for (int q = 0; q < kRingK; ++q) {
            const int i = tid + q * NT;
            if (i < j0 * (kDim / 4)) ring_k[q] = ld4(recb + (int64_t)T * kDim + 4 * i);
        }
        if constexpr (CH) {   // the pending positions' per-channel decays
#pragma unroll
            for (int q = 0; q < kRingK; ++q) {
                const int i = tid + q * NT;
                if (i < j0 * (kDim / 4)) ring_a[q] = ld4(recb + 2 * (int64_t)T * kDim + 4 * i);
            }
        } else {
            if (tid < j0) ring_g = recb[2 * (int64_t)T * kDim + tid];
        }
    }
    const StateT* head = static_cast<const StateT*>(p.state) + ((int64_t)slot * p.hv + hv) * kHeadElems;
    f32x4 h[R][4];
    TileIO<StateT, R>::load(head, row0, grp, lane8, h);

    // ---- stage the window in LDS ----
    if constexpr (!SNAP) {
#pragma unroll
        for (int q = 0; q < kRingD; ++q) {
            const int i = tid + q * NT;
            if (i < j0 * kRowQ) {
                const int t = i / kRowQ;
                st4(L.vd + t * kRowsPerWg + 4 * (i - t * kRowQ), ring_d[q]);
            }
        }
#pragma unroll
        for (int q = 0; q < kRingK; ++q) {
            const int i = tid + q * NT;
            if (i < j0 * (kDim / 4)) st4(L.khat + 4 * i, ring_k[q]);
        }
        if constexpr (CH) {
#pragma unroll
            for (int q = 0; q < kRingK; ++q) {
                const int i = tid + q * NT;
                if (i < j0 * (kDim / 4)) st4(L.al + 4 * i, ring_a[q]);
            }
        } else {
            if (tid < j0) L.g[tid] = ring_g;
        }
    }
    if constexpr (CH) {   // the window's per-channel decays, and their record (lead chunk)
#pragma unroll
        for (int q = 0; q < kAChunks; ++q) {
            const int i = tid + q * NT;
            if (i < w * (kDim / 4)) {
                const int t = i / (kDim / 4);
                const int off = (j0 + t) * kDim + 4 * (i - t * (kDim / 4));
                const f32x4 al = f32x4{expf(win_a[q].x), expf(win_a[q].y), expf(win_a[q].z),
                                       expf(win_a[q].w)};
                st4(L.al + off, al);
                if (!SNAP && lead) st4(recb + 2 * (int64_t)T * kDim + off, al);
            }
        }
    }
    for (int jb = jb0; jb < 3 * w; jb += NT / 16) {
        const int t = jb / 3;
        const int kind = jb - 3 * t;
        const u32x4 raw = jb == jb0 ? raw0 : *reinterpret_cast<const u32x4*>(job_src(jb) + 8 * lane16);
        float x[8] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y),
                      bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w)};
        const int off = (j0 + t) * kDim + 8 * lane16;
        if (!SNAP && lead && p.payload && kind != 0) {
            // payload record: the raw key (kind 1) or value (kind 2) bits
            uint16_t* rp = reinterpret_cast<uint16_t*>(recb) + (kind == 2 ? (int64_t)T * kDim : 0) + off;
            *reinterpret_cast<u32x4*>(rp) = raw;
        }
        if (kind == 2) {          // values: the owned rows only
            const int c = 8 * lane16 - row0;
            if (c >= 0 && c < kRowsPerWg) {
                float* vp = L.vd + (j0 + t) * kRowsPerWg + c;
                st4(vp, f32x4{x[0], x[1], x[2], x[3]});
                st4(vp + 4, f32x4{x[4], x[5], x[6], x[7]});
            }
            continue;
        }
        l2norm_row16(x);
        if (kind == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = x[i] * p.scale;
            st4(L.qt + off, f32x4{x[0], x[1], x[2], x[3]});
            st4(L.qt + off + 4, f32x4{x[4], x[5], x[6], x[7]});
        } else {
            st4(L.khat + off, f32x4{x[0], x[1], x[2], x[3]});
            st4(L.khat + off + 4, f32x4{x[4], x[5], x[6], x[7]});
            if (!SNAP && lead && !p.payload) {
                float* rk = recb + (int64_t)T * kDim + off;
                st4(rk, f32x4{x[0], x[1], x[2], x[3]});
                st4(rk + 4, f32x4{x[4], x[5], x[6], x[7]});
            }
        }
    }
    for (int t = tid; t < w; t += NT) {
        float av = a_in, bv = b_in;
        if (t != tid) {          // windows longer than the workgroup (not reachable at T <= 16)
            const int64_t tok = (int64_t)ts + t;
            if constexpr (!CH) av = p.a_log[tok * p.g_ts + hv];
            bv = p.beta[tok * p.g_ts + hv];
        }
        if constexpr (CH) {      // the decays are per channel (staged above); beta as given
            L.be[j0 + t] = bv;
            continue;
        }
        float g, be;
        if (p.raw_gates) {
            // g = exp(-exp(A_log) softplus(a + dt_bias)), beta = sigmoid(b)
            const float x = av + dtb_in;
            const float sp = x > kSoftplusLinear ? x : log1pf(expf(x));
            g = expf(-expf(alog_in) * sp);
            be = 1.0f / (1.0f + expf(-bv));
        } else {
            g = expf(av);
            be = bv;
        }
        L.g[j0 + t] = g;
        L.be[j0 + t] = be;
        if (!SNAP && lead) {
            if (p.payload) {      // gate and beta after the bf16 key and value fields
                recb[(int64_t)T * kDim + j0 + t] = g;
                recb[(int64_t)T * (kDim + 1) + j0 + t] = be;
            } else {
                recb[2 * (int64_t)T * kDim + j0 + t] = g;
            }
        }
    }
    __syncthreads();

    // ---- per-item scalars: G(0, p+1) and the coefficients of earlier corrections ----
    // Window position p has 2p + 1 dot-product jobs: (k_j . k_p) for j < p, then
    // (k_j . q_p) for j <= p; jobs of p start at p^2 - j0^2.
    const int njobs = P * P - j0 * j0;
    float gv[TT];                         // the decays, read from LDS once, independently
#pragma unroll
    for (int m = 0; m < TT; m += 4) {
        const f32x4 g4 = ld4(L.g + m);
        gv[m] = g4.x; gv[m + 1] = g4.y; gv[m + 2] = g4.z; gv[m + 3] = g4.w;
    }
    for (int jb = tid >> 4; jb < njobs; jb += NT / 16) {
        int pp = j0;
        while ((pp + 1) * (pp + 1) - j0 * j0 <= jb) ++pp;
        const int rem = jb - (pp * pp - j0 * j0);
        const bool is_q = rem >= pp;
        const int j = is_q ? rem - pp : rem;
        const float* a = L.khat + j * kDim + 8 * lane16;
        const float* c = (is_q ? L.qt : L.khat) + pp * kDim + 8 * lane16;
        f32x4 a0 = ld4(a), a1 = ld4(a + 4);
        const f32x4 c0 = ld4(c), c1 = ld4(c + 4);
        if constexpr (CH) {
            // k_j weighted channel by channel by the decays of positions j+1 .. pp
            f32x4 w0 = {1.f, 1.f, 1.f, 1.f}, w1 = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
            for (int m = 1; m < TT; ++m)
                if (m > j && m <= pp) {
                    const f32x4 x0 = ld4(L.al + m * kDim + 8 * lane16), x1 = ld4(L.al + m * kDim + 8 * lane16 + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        w0[e] = w0[e] * x0[e];
                        w1[e] = w1[e] * x1[e];
                    }
                }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a0[e] = a0[e] * w0[e];
                a1[e] = a1[e] * w1[e];
            }
        }
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) dot = __builtin_fmaf(a0[e], c0[e], dot);
#pragma unroll
        for (int e = 0; e < 4; ++e) dot = __builtin_fmaf(a1[e], c1[e], dot);
        dot = sum16(dot);
        if constexpr (CH) {
            if (lane16 == 0) (is_q ? L.cb : L.ca)[j * TT + pp] = dot;
        } else {
            float gam = 1.f;              // g_{j+1} ... g_pp, in that order
#pragma unroll
            for (int m = 1; m < TT; ++m)
                if (m > j && m <= pp) gam = gam * gv[m];
            if (lane16 == 0) (is_q ? L.cb : L.ca)[j * TT + pp] = gam * dot;
        }
    }
    if constexpr (CH) {
        // the vectors the checkpoint meets: k_p and q_p scaled channel by
        // channel by the decays of positions 0 .. p, in that order (verify
        // overwrites the staged keys and queries once every coefficient job
        // has read them)
        if constexpr (!SNAP) __syncthreads();
        float* const kdst = SNAP ? L.kx : L.khat;
        float* const qdst = SNAP ? L.qx : L.qt;
        for (int i = tid; i < w * (kDim / 4); i += NT) {
            const int pp = j0 + i / (kDim / 4);
            const int c = 4 * (i % (kDim / 4));
            f32x4 gam = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
            for (int m = 0; m < TT; ++m)
                if (m <= pp) {
                    const f32x4 x = ld4(L.al + m * kDim + c);
#pragma unroll
                    for (int e = 0; e < 4; ++e) gam[e] = gam[e] * x[e];
                }
            const f32x4 kv = ld4(L.khat + pp * kDim + c), qv = ld4(L.qt + pp * kDim + c);
            st4(kdst + pp * kDim + c, f32x4{gam.x * kv.x, gam.y * kv.y, gam.z * kv.z, gam.w * kv.w});
            st4(qdst + pp * kDim + c, f32x4{gam.x * qv.x, gam.y * qv.y, gam.z * qv.z, gam.w * qv.w});
        }
        for (int t = tid; t < w; t += NT) L.g0[j0 + t] = 1.f;
    } else {
        for (int t = tid; t < w; t += NT) {
            float gam = 1.f;              // g_0 ... g_{j0+t}, in that order
#pragma unroll
            for (int m = 0; m < TT; ++m)
                if (m <= j0 + t) gam = gam * gv[m];
            L.g0[j0 + t] = gam;
        }
    }
    __syncthreads();

    // ---- the window, position by position (unrolled over the capacity TT;
    // the corrections of the owned rows stay in registers) ----
    // Each lane finishes rows rm, rm + 2, ... (RH of them): lanes 0-3 of the
    // group the even rows of the group's R, lanes 4-7 the odd ones.
    constexpr int RH = R / 2;
    const bool hi = (lane8 & 4) != 0;
    const int rm = R * grp + (hi ? 1 : 0);   // relative to row0
    float dreg[TT][RH];
#pragma unroll
    for (int pp = 0; pp < TT; ++pp) {
        if (pp < j0) {                 // ring position: its recorded correction
#pragma unroll
            for (int m = 0; m < RH; ++m) dreg[pp][m] = L.vd[pp * kRowsPerWg + rm + 2 * m];
            continue;
        }
        if (pp >= P) break;
        const float g0 = L.g0[pp];
        float pk[RH];
        tile_dot_split<StateT, R>(h, (CH && SNAP ? L.kx : L.khat) + pp * kDim, lane8, hi, pk);
        float u[RH];
#pragma unroll
        for (int m = 0; m < RH; ++m) u[m] = g0 * pk[m];
#pragma unroll
        for (int j = 0; j < pp; ++j) {
            const float cf = L.ca[j * TT + pp];
#pragma unroll
            for (int m = 0; m < RH; ++m) u[m] = __builtin_fmaf(cf, dreg[j][m], u[m]);
        }
        const float be = L.be[pp];
#pragma unroll
        for (int m = 0; m < RH; ++m) dreg[pp][m] = be * (L.vd[pp * kRowsPerWg + rm + 2 * m] - u[m]);
#pragma unroll
        for (int m = 0; m < RH; ++m) L.dw[pp * kRowsPerWg + rm + 2 * m] = dreg[pp][m];  // same value in 4 lanes

        float pq[RH];
        tile_dot_split<StateT, R>(h, (CH && SNAP ? L.qx : L.qt) + pp * kDim, lane8, hi, pq);
        float o[RH];
#pragma unroll
        for (int m = 0; m < RH; ++m) o[m] = g0 * pq[m];
#pragma unroll
        for (int j = 0; j <= pp; ++j) {
            const float cf = L.cb[j * TT + pp];
#pragma unroll
            for (int m = 0; m < RH; ++m) o[m] = __builtin_fmaf(cf, dreg[j][m], o[m]);
        }
#pragma unroll
        for (int m = 0; m < RH; ++m) L.ob[pp * kRowsPerWg + rm + 2 * m] = o[m];   // same value in 4 lanes
    }
    __syncthreads();

    // ---- outputs and corrections of the owned rows, written out coalesced and
    // nontemporal (nothing in this launch reads them back; streaming them past
    // the caches measured 1-2% faster) ----
    {
        constexpr int kRow4 = kRowsPerWg / 4;
        for (int i = tid; i < w * kRow4; i += NT) {
            const int t = i / kRow4;
            const int c = 4 * (i - t * kRow4);
            const f32x4 ov = ld4(L.ob + (j0 + t) * kRowsPerWg + c);
            const int64_t oo = ((int64_t)ts + t) * p.o_ts + (int64_t)hv * p.o_hs + row0 + c;
            if (p.out_bf16)
                *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + oo) =
                    u32x2{pack_bf16(ov.x, ov.y), pack_bf16(ov.z, ov.w)};
            else
                st4_nt(static_cast<float*>(p.out) + oo, ov);
            if (!SNAP && !p.payload) st4_nt(recb + (j0 + t) * kDim + row0 + c, ld4(L.dw + (j0 + t) * kRowsPerWg + c));
        }
    }

    // ---- native baseline: materialise and write S_1..S_w ----
    if constexpr (SNAP) {
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            if (t >= w) break;
            const float g = L.g[t];
            f32x4 kh[4], dc[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                kh[c] = ld4(L.khat + t * kDim + tcol<StateT>(lane8, c));
                dc[c] = CH ? ld4(L.al + t * kDim + tcol<StateT>(lane8, c)) : f32x4{g, g, g, g};
            }
            float dr[R];              // both rows of each pair, from the two halves
#pragma unroll
            for (int m = 0; m < RH; ++m) {
                const float other = dpp<kDppRowHalfMirror>(dreg[t][m]);
                dr[2 * m] = hi ? other : dreg[t][m];
                dr[2 * m + 1] = hi ? dreg[t][m] : other;
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float d = dr[r];
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int e = 0; e < 4; ++e) h[r][c][e] = __builtin_fmaf(d, kh[c][e], h[r][c][e] * dc[c][e]);
            }
            StateT* sn = static_cast<StateT*>(p.snap) + (((int64_t)b * p.hv + hv) * T + t) * kHeadElems;
            TileIO<StateT, R>::store(sn, row0, grp, lane8, h);
        }
    }
}

template <typename StateT, bool SNAP, int R, int NT, int TT, bool CH>
hipError_t launch_tt(const VerifyParams& p, hipStream_t s)
{
    VerifyParams args = p;
    void* kargs[] = {&args};
    const unsigned chunks = kDim / (NT / 8 * R);
    const unsigned grid = (unsigned)(p.num_rows * p.hv) * chunks;
    const size_t lds = sizeof(float) * Lds<TT, NT / 8 * R, CH, SNAP>::kFloats;
    return hipLaunchKernel(reinterpret_cast<const void*>(&verify_kernel<StateT, SNAP, R, NT, TT, CH>),
                           dim3(grid), dim3(NT), kargs, lds, s);
}

// The smallest compile-time window capacity that holds the record capacity.
template <typename StateT, bool SNAP, bool CH>
hipError_t launch_ch(const VerifyParams& p, hipStream_t s)
{
    constexpr int R = kVerifyRowsPerThread, NT = kVerifyThreads;
    if (p.T <= 4) return launch_tt<StateT, SNAP, R, kVerifyThreadsShort, 4, CH>(p, s);
    if (p.T <= 8) return launch_tt<StateT, SNAP, R, NT, 8, CH>(p, s);
    return launch_tt<StateT, SNAP, R, NT, kMaxRecTokens, CH>(p, s);
}

template <typename StateT, bool SNAP>
hipError_t launch(const VerifyParams& p, hipStream_t s)
{
    return p.channel ? launch_ch<StateT, SNAP, true>(p, s) : launch_ch<StateT, SNAP, false>(p, s);
}

}  // namespace

hipError_t launch_verify(const VerifyParams& p, bool bf16_state, hipStream_t s)
{
    return bf16_state ? launch<uint16_t, false>(p, s) : launch<float, false>(p, s);
}

hipError_t launch_native_window(const VerifyParams& p, bool bf16_state, hipStream_t s)
{
    return bf16_state ? launch<uint16_t, true>(p, s) : launch<float, true>(p, s);
}

}  // namespace gdn
