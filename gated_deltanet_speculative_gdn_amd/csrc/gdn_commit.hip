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
// One launch, one workgroup of four wave64s per (layer, row, value head). The
// workgroup reads its whole source head (64 KiB fp32 / 32 KiB bf16) into
// registers with fully coalesced 16-byte loads -- thread t owns 16-byte pieces
// t + 256*i, so each load instruction of the workgroup covers 4 KiB of
// contiguous memory -- stages the n records in LDS, replays n tokens
// elementwise (no reductions), then stores the final state and, in align mode,
// the boundary state kept in a second register tile. Because every thread
// reads all of its source elements before its first store and writes only the
// elements it read, a destination or boundary slot equal to the source slot is
// safe; the pages' read-after-overwrite race between programs cannot occur.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

#pragma clang fp contract(off)

namespace gdn {
namespace {

// Ownership of the elements of one head by thread t:
//   fp32: 16 pieces of 4 floats, piece f = t + 256*i: row f/32, columns 4*(f%32)..+3.
//   bf16: 8 pieces of 8 values, piece f = t + 256*i: row f/16, columns 8*(f%16)..+7.
template <typename StateT> struct HeadIO;

template <> struct HeadIO<float> {
    static constexpr int kPieces = 16;
    typedef f32x4 Raw;
    __device__ static void load(const float* head, int t, f32x4 (&h)[16]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) h[i] = ld4(head + 4 * (t + kThreads * i));
    }
    template <bool NT>
    __device__ static void store(float* head, int t, const f32x4 (&h)[16]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if constexpr (NT) st4_nt(head + 4 * (t + kThreads * i), h[i]);
            else st4(head + 4 * (t + kThreads * i), h[i]);
        }
    }
    // row of element e of piece i, and the column of element 0
    __device__ static int row(int t, int i) { return (t + kThreads * i) >> 5; }
    __device__ static int col0(int t) { return 4 * (t & 31); }
};

template <> struct HeadIO<uint16_t> {
    static constexpr int kPieces = 8;
    // the same 64 values per thread, held as 16 f32x4: h[2i] = columns +0..3, h[2i+1] = +4..7
    __device__ static void load(const uint16_t* head, int t, f32x4 (&h)[16]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(head + 8 * (t + kThreads * i));
            h[2 * i] = f32x4{bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y)};
            h[2 * i + 1] = f32x4{bf16_lo(x.z), bf16_hi(x.z), bf16_lo(x.w), bf16_hi(x.w)};
        }
    }
    template <bool NT>
    __device__ static void store(uint16_t* head, int t, const f32x4 (&h)[16]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 a = h[2 * i], c = h[2 * i + 1];
            const u32x4 x{pack_bf16(a.x, a.y), pack_bf16(a.z, a.w), pack_bf16(c.x, c.y),
                          pack_bf16(c.z, c.w)};
            u32x4* dst = reinterpret_cast<u32x4*>(head + 8 * (t + kThreads * i));
            if constexpr (NT) __builtin_nontemporal_store(x, dst);
            else *dst = x;
        }
    }
    __device__ static int row(int t, int i) { return (t + kThreads * i) >> 4; }
    __device__ static int col0(int t) { return 8 * (t & 15); }
};

template <typename StateT, bool ALIGN>
__global__ void __launch_bounds__(kThreads) commit_kernel(CommitParams p)
{
    extern __shared__ float lds[];
    const int T = p.T;
    float* d_l = lds;                 // [n][128] corrections
    float* k_l = lds + T * kDim;      // [n][128] normalised keys
    float* g_l = lds + 2 * T * kDim;  // [n] decays

    const int64_t wg = blockIdx.x;
    const int hv = (int)(wg % p.hv);
    const int64_t lb = wg / p.hv;
    const int b = (int)(lb % p.num_rows);
    const int layer = (int)(lb / p.num_rows);

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
    int err = 0;
    if (n < 0 || n > T || dst < 0) err |= kRowN;
    if (src >= p.num_slots || dst >= p.num_slots) err |= kRowSlot;
    if (rs < 0 || rs >= p.num_rec_slots) err |= kRowRec;
    if (ALIGN && bl != 0 && (bl < 0 || bl >= n || bs < 0 || bs >= p.num_slots)) err |= kRowBnd;
    if (err) {
        if (threadIdx.x == 0 && hv == 0 && layer == 0 && p.err) atomicOr(p.err, err);
        return;
    }
    const bool write_bnd = ALIGN && bl > 0 && bs != dst;

    const int t = threadIdx.x;
    StateT* pool = static_cast<StateT*>(p.state[layer]);
    const int64_t head_off = (int64_t)p.hv * kHeadElems;
    f32x4 h[16];
    HeadIO<StateT>::load(pool + src * head_off + (int64_t)hv * kHeadElems, t, h);

    // ---- the n records into LDS ----
    const float* recb = p.rec[layer] + ((int64_t)rs * p.hv + hv) * p.rec_stride;
    for (int i = t; i < n * (kDim / 4); i += kThreads) {
        st4(d_l + 4 * i, ld4(recb + 4 * i));
        st4(k_l + 4 * i, ld4(recb + (int64_t)T * kDim + 4 * i));
    }
    if (t < n) g_l[t] = recb[2 * (int64_t)T * kDim + t];
    __syncthreads();

    // ---- replay: h = fma(delta_t[row], k_hat_t[col], h * g_t) ----
    f32x4 hb[ALIGN ? 16 : 1];
    const int c0 = HeadIO<StateT>::col0(t);
    for (int tt = 0; tt < n; ++tt) {
        const float g = g_l[tt];
        if constexpr (sizeof(StateT) == 4) {
            const f32x4 kh = ld4(k_l + tt * kDim + c0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float d = d_l[tt * kDim + HeadIO<StateT>::row(t, i)];
#pragma unroll
                for (int e = 0; e < 4; ++e) h[i][e] = __builtin_fmaf(d, kh[e], h[i][e] * g);
            }
        } else {
            const f32x4 kh0 = ld4(k_l + tt * kDim + c0);
            const f32x4 kh1 = ld4(k_l + tt * kDim + c0 + 4);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float d = d_l[tt * kDim + HeadIO<StateT>::row(t, i)];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[2 * i][e] = __builtin_fmaf(d, kh0[e], h[2 * i][e] * g);
                    h[2 * i + 1][e] = __builtin_fmaf(d, kh1[e], h[2 * i + 1][e] * g);
                }
            }
        }
        if constexpr (ALIGN) {
            if (tt + 1 == bl) {
#pragma unroll
                for (int i = 0; i < 16; ++i) hb[i] = h[i];
            }
        }
    }

    // ---- final state first, then the boundary state ----
    HeadIO<StateT>::template store<true>(pool + dst * head_off + (int64_t)hv * kHeadElems, t, h);
    if constexpr (ALIGN) {
        if (write_bnd)
            HeadIO<StateT>::template store<true>(pool + bs * head_off + (int64_t)hv * kHeadElems,
                                                 t, hb);
    }
}

// Native baseline: copy the snapshot of the last accepted token into the slot.
template <typename StateT>
__global__ void __launch_bounds__(kThreads) accept_kernel(AcceptParams p)
{
    const int64_t wg = blockIdx.x;
    const int hv = (int)(wg % p.hv);
    const int64_t lb = wg / p.hv;
    const int b = (int)(lb % p.num_rows);
    const int layer = (int)(lb / p.num_rows);
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

template <typename StateT, bool ALIGN>
hipError_t launch_c(const CommitParams& p, hipStream_t s)
{
    CommitParams args = p;
    void* kargs[] = {&args};
    const uint64_t grid = (uint64_t)p.num_layers * p.num_rows * p.hv;
    return hipLaunchKernel(reinterpret_cast<const void*>(&commit_kernel<StateT, ALIGN>),
                           dim3((unsigned)grid), dim3(kThreads), kargs, commit_lds_bytes(p.T), s);
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
    if (bf16_state) return align ? launch_c<uint16_t, true>(p, s) : launch_c<uint16_t, false>(p, s);
    return align ? launch_c<float, true>(p, s) : launch_c<float, false>(p, s);
}

hipError_t launch_native_accept(const AcceptParams& p, bool bf16_state, hipStream_t s)
{
    return bf16_state ? launch_a<uint16_t>(p, s) : launch_a<float>(p, s);
}

}  // namespace gdn
