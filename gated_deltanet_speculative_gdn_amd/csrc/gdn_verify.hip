// gdn_verify.hip -- verify from a read-only checkpoint, and the native
// snapshot-every-token baseline, for gfx950.
//
// Method: vLLM PR "[Spec Decode][Qwen4Exp] RecoverSSM for Qwen GDN and the PLE
// short conv", Purpose (verify runs the draft window from the checkpoint,
// writes the per-token outputs and an fp32 record of correction, normalised key
// and gate, never the state) and Test Result (the record holds the decay that
// was multiplied in); the rule itself is the gated delta rule of "Gated Delta
// Networks" (Yang, Kautz, Hatamizadeh, ICLR 2025). Ring mode (records of
// earlier single-token steps replayed in registers before the window) follows
// the 16-token replay buffer of lmdeploy PR #5028 (Performance test settings).
//
// One workgroup of four wave64s per (row, value head). The 128x128 fp32 head
// lives in registers, 64 values per lane: lane l holds rows 4*(l/8) + r and
// columns 4*(l%8) + 32*c + e (r, c, e = 0..3), so each of its 16 vector loads
// reads one 16-byte piece and eight neighbouring lanes read a whole 128-byte
// row segment. The two length-128 reductions per token (h'k_hat and h q_tilde)
// are 16 fmas in the lane followed by a three-step DPP sum over the eight lanes
// of a row group -- no LDS traffic and no barrier inside the token loop. The
// window's normalised q, k, the values, gates and ring records are staged in
// LDS once, before the loop.
//
// The native baseline is the same template with SNAP = true: identical
// arithmetic, plus a store of the state after every token. Verify outputs and
// records are therefore bit-identical to the baseline's, and the commit's
// replay of them reproduces the baseline's states bit for bit.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

#pragma clang fp contract(off)

namespace gdn {
namespace {

// Register tile: h[r][c] holds row 4*grp + r, columns 4*lane8 + 32*c .. +3.
template <typename StateT> struct TileIO;

template <> struct TileIO<float> {
    __device__ static void load(const float* head, int grp, int lane8, f32x4 (&h)[4][4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                h[r][c] = ld4(head + (4 * grp + r) * kDim + 4 * lane8 + 32 * c);
    }
    __device__ static void store(float* head, int grp, int lane8, const f32x4 (&h)[4][4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                st4(head + (4 * grp + r) * kDim + 4 * lane8 + 32 * c, h[r][c]);
    }
};

// bf16 pool: the same element ownership, 8-byte loads (four bf16 values).
template <> struct TileIO<uint16_t> {
    __device__ static void load(const uint16_t* head, int grp, int lane8, f32x4 (&h)[4][4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x2 x = *reinterpret_cast<const u32x2*>(
                    head + (4 * grp + r) * kDim + 4 * lane8 + 32 * c);
                h[r][c] = f32x4{bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y)};
            }
    }
    __device__ static void store(uint16_t* head, int grp, int lane8, const f32x4 (&h)[4][4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f32x4 v = h[r][c];
                *reinterpret_cast<u32x2*>(head + (4 * grp + r) * kDim + 4 * lane8 + 32 * c) =
                    u32x2{pack_bf16(v.x, v.y), pack_bf16(v.z, v.w)};
            }
    }
};

template <typename StateT, bool SNAP>
__global__ void __launch_bounds__(kThreads) verify_kernel(VerifyParams p)
{
    extern __shared__ float lds[];
    const int T = p.T;
    float* khat_l = lds;                  // [T][128] normalised keys (ring and window)
    float* vd_l = lds + T * kDim;         // [T][128] ring: corrections; window: values
    float* qt_l = lds + 2 * T * kDim;     // [T][128] normalised, scaled queries
    float* g_l = lds + 3 * T * kDim;      // [T] decays
    float* be_l = g_l + T;                // [T] write strengths

    const int b = blockIdx.x / p.hv;
    const int hv = blockIdx.x - b * p.hv;

    // ---- row decode: a null slot or an empty window is padding ----
    const int slot = p.state_slot[b];
    const int w = p.win_len[b];
    if (slot < 0 || w == 0) return;
    const int ts = p.tok_start[b];
    int j0 = 0, rs = 0;
    if constexpr (!SNAP) {
        j0 = p.rec_base ? p.rec_base[b] : 0;
        rs = p.rec_slot[b];
    }
    int err = 0;
    if (slot >= p.num_slots) err |= kRowSlot;
    if (w < 0 || j0 < 0 || (int64_t)j0 + w > T || ts < 0 || (int64_t)ts + w > p.num_tokens)
        err |= kRowWin;
    if (!SNAP && (rs < 0 || rs >= p.num_rec_slots)) err |= kRowRec;
    if (err) {
        if (threadIdx.x == 0 && p.err) atomicOr(p.err, err);
        return;
    }

    const int tid = threadIdx.x;
    const int lane8 = tid & 7;
    const int grp = tid >> 3;

    // ---- checkpoint head into registers (issued first, consumed after the barrier) ----
    const StateT* head = static_cast<const StateT*>(p.state) + ((int64_t)slot * p.hv + hv) * kHeadElems;
    f32x4 h[4][4];
    TileIO<StateT>::load(head, grp, lane8, h);

    float* recb = nullptr;
    if constexpr (!SNAP) {
        recb = p.rec + ((int64_t)rs * p.hv + hv) * p.rec_stride;
        // pending ring records (positions 0 .. j0-1) into LDS
        for (int i = tid; i < j0 * (kDim / 4); i += kThreads) {
            st4(vd_l + 4 * i, ld4(recb + 4 * i));
            st4(khat_l + 4 * i, ld4(recb + (int64_t)T * kDim + 4 * i));
        }
        for (int i = tid; i < j0; i += kThreads) g_l[i] = recb[2 * (int64_t)T * kDim + i];
    }

    // ---- window vectors: three jobs per token (q, k, v), one 16-lane DPP row each ----
    const int lane16 = tid & 15;
    const int hk = hv / p.group;
    for (int jb = tid >> 4; jb < 3 * w; jb += kThreads / 16) {
        const int t = jb / 3;
        const int kind = jb - 3 * t;
        const int64_t tok = (int64_t)ts + t;
        const int pos = j0 + t;
        const uint16_t* src = kind == 0 ? p.q + tok * p.q_ts + hk * p.q_hs
                            : kind == 1 ? p.k + tok * p.k_ts + hk * p.k_hs
                                        : p.v + tok * p.v_ts + hv * p.v_hs;
        const u32x4 raw = *reinterpret_cast<const u32x4*>(src + 8 * lane16);
        float x[8] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y),
                      bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w)};
        const int off = pos * kDim + 8 * lane16;
        if (kind == 2) {
            st4(vd_l + off, f32x4{x[0], x[1], x[2], x[3]});
            st4(vd_l + off + 4, f32x4{x[4], x[5], x[6], x[7]});
            continue;
        }
        float ssq = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ssq = __builtin_fmaf(x[i], x[i], ssq);
        ssq = sum16(ssq);
        const float inv = 1.0f / __builtin_sqrtf(ssq + kNormEps);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = x[i] * inv;
        if (kind == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = x[i] * p.scale;
            st4(qt_l + off, f32x4{x[0], x[1], x[2], x[3]});
            st4(qt_l + off + 4, f32x4{x[4], x[5], x[6], x[7]});
        } else {
            st4(khat_l + off, f32x4{x[0], x[1], x[2], x[3]});
            st4(khat_l + off + 4, f32x4{x[4], x[5], x[6], x[7]});
            if constexpr (!SNAP) {
                float* rk = recb + (int64_t)T * kDim + off;
                st4(rk, f32x4{x[0], x[1], x[2], x[3]});
                st4(rk + 4, f32x4{x[4], x[5], x[6], x[7]});
            }
        }
    }
    for (int t = tid; t < w; t += kThreads) {
        const int64_t tok = (int64_t)ts + t;
        const float g = expf(p.a_log[tok * p.g_ts + hv]);
        g_l[j0 + t] = g;
        be_l[j0 + t] = p.beta[tok * p.g_ts + hv];
        if constexpr (!SNAP) recb[2 * (int64_t)T * kDim + j0 + t] = g;
    }
    __syncthreads();

    // ---- ring: replay the pending records onto the checkpoint ----
    for (int pos = 0; pos < j0; ++pos) {
        const float g = g_l[pos];
        f32x4 kh[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) kh[c] = ld4(khat_l + pos * kDim + 4 * lane8 + 32 * c);
        const f32x4 d = ld4(vd_l + pos * kDim + 4 * grp);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    h[r][c][e] = __builtin_fmaf(d[r], kh[c][e], h[r][c][e] * g);
    }

    // ---- the window, token by token ----
    for (int t = 0; t < w; ++t) {
        const int pos = j0 + t;
        const float g = g_l[pos];
        const float be = be_l[pos];
        f32x4 kh[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) kh[c] = ld4(khat_l + pos * kDim + 4 * lane8 + 32 * c);
        const f32x4 vv = ld4(vd_l + pos * kDim + 4 * grp);

        // h' = g h, u = h' k_hat
        float u[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[r][c][e] = h[r][c][e] * g;
                    acc = __builtin_fmaf(h[r][c][e], kh[c][e], acc);
                }
            u[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) u[r] = sum8(u[r]);

        // delta = beta (v - u);  h = fma(delta, k_hat, h')
        f32x4 d;
#pragma unroll
        for (int r = 0; r < 4; ++r) d[r] = be * (vv[r] - u[r]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    h[r][c][e] = __builtin_fmaf(d[r], kh[c][e], h[r][c][e]);

        // o = h q_tilde
        f32x4 qt[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) qt[c] = ld4(qt_l + pos * kDim + 4 * lane8 + 32 * c);
        f32x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(h[r][c][e], qt[c][e], acc);
            o[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = sum8(o[r]);

        if (lane8 == 0) {
            st4(p.out + ((int64_t)ts + t) * p.o_ts + hv * p.o_hs + 4 * grp, o);
            if constexpr (!SNAP) st4(recb + pos * kDim + 4 * grp, d);
        }
        if constexpr (SNAP) {
            StateT* sn = static_cast<StateT*>(p.snap) +
                         (((int64_t)b * p.hv + hv) * T + t) * kHeadElems;
            TileIO<StateT>::store(sn, grp, lane8, h);
        }
    }
}

template <typename StateT, bool SNAP>
hipError_t launch(const VerifyParams& p, hipStream_t s)
{
    VerifyParams args = p;
    void* kargs[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void*>(&verify_kernel<StateT, SNAP>),
                           dim3((unsigned)(p.num_rows * p.hv)), dim3(kThreads), kargs,
                           verify_lds_bytes(p.T), s);
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
