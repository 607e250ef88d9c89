// gdn_plan.hip -- align-mode commit plan, one thread per row, and the debug
// check of a commit's slot preconditions (gdn_check_slots), for gfx950.
//
// Method: vLLM PR "[Spec Decode][Qwen4Exp] RecoverSSM for Qwen GDN and the PLE
// short conv" -- Purpose (align mode writes the block-boundary state as well
// as the final state), Commits item 3 (a window whose accepted tokens end
// exactly on a block boundary commits into the block of its last token) and
// item 6 (a boundary state may land in the source slot; a boundary whose slot
// is the final slot is not written). A state covering m tokens lives in block
// column (m - 1) / B. Closed form used here, with r = p0 mod B:
//   source column (p0 - 1) / B, final column (p0 + n - 1) / B, and the first
//   block boundary inside the window after t_b = B - r tokens (B when r = 0);
//   it is a boundary-state write iff t_b < n, into column (p0 + t_b - 1) / B.
//   A second boundary (t_b + B < n) is an error: blocks must hold a window.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {
namespace {

__global__ void __launch_bounds__(kThreads) align_plan_kernel(PlanParams p)
{
    const int b = blockIdx.x * kThreads + threadIdx.x;
    if (b >= p.num_rows) return;
    const int p0 = p.p0[b];
    const int n = p.n[b];
    const int32_t* tb = p.table + (int64_t)b * p.table_stride;
    const int B = p.block;
    int err = 0;
    int src = -1, dst = -1, bl = 0, bs = -1;
    if (p0 < 1) err |= kRowPos;
    if (n < 0 || n > p.max_n) err |= kRowN;
    if (!err) {
        const int64_t cs = ((int64_t)p0 - 1) / B;
        if (cs >= p.cols || tb[cs] < 0) err |= kRowTable;
        else src = tb[cs];
    }
    if (!err && n > 0) {
        const int64_t cd = ((int64_t)p0 + n - 1) / B;
        const int r = (int)(p0 % B);
        const int t_b = r ? B - r : B;
        if (t_b < n && (int64_t)t_b + B < n) err |= kRowBnd;      // two boundaries
        if (!err && (cd >= p.cols || tb[cd] < 0)) err |= kRowTable;
        if (!err) dst = tb[cd];
        if (!err && t_b < n) {
            const int64_t cb = ((int64_t)p0 + t_b - 1) / B;
            if (cb >= p.cols || tb[cb] < 0) err |= kRowTable;
            else if (tb[cb] != dst) { bl = t_b; bs = tb[cb]; }
        }
    }
    if (err) {
        src = dst = bs = -1;
        bl = 0;
        if (p.err) atomicOr(p.err, err);
    }
    p.src[b] = src;
    p.dst[b] = dst;
    p.bnd_len[b] = bl;
    p.bnd_slot[b] = bs;
}

// Slot-alias check of one commit (a debug aid): thread a compares its live row
// with every other live row. Written slots: the destination and a boundary
// slot other than it; read slot: the source; a record slot read by one row
// only. Any overlap across two rows sets the alias bit.
struct SlotCheckParams {
    const int32_t *src, *dst, *rec, *n, *bnd_len, *bnd_slot;
    int32_t* err;
    int32_t num_rows;
};

__device__ __forceinline__ void row_slots(const SlotCheckParams& p, int b, bool& live, int& src,
                                          int& w0, int& w1, int& rec)
{
    src = p.src[b];
    live = p.n[b] > 0 && src >= 0;
    w0 = p.dst[b];
    w1 = -1;
    if (p.bnd_len && p.bnd_len[b] > 0 && p.bnd_slot[b] != w0) w1 = p.bnd_slot[b];
    rec = p.rec ? p.rec[b] : -1;
}

__global__ void __launch_bounds__(kThreads) slot_check_kernel(SlotCheckParams p)
{
    const int a = blockIdx.x * kThreads + threadIdx.x;
    if (a >= p.num_rows) return;
    bool la;
    int sa, wa0, wa1, ra;
    row_slots(p, a, la, sa, wa0, wa1, ra);
    if (!la) return;
    bool alias = false;
    for (int b = 0; b < p.num_rows && !alias; ++b) {
        if (b == a) continue;
        bool lb;
        int sb, wb0, wb1, rb;
        row_slots(p, b, lb, sb, wb0, wb1, rb);
        if (!lb) continue;
        const bool ww = (wa0 >= 0 && (wa0 == wb0 || wa0 == wb1)) || (wa1 >= 0 && (wa1 == wb0 || wa1 == wb1));
        const bool wr = (wa0 >= 0 && wa0 == sb) || (wa1 >= 0 && wa1 == sb);
        const bool rr = ra >= 0 && ra == rb;
        alias = ww || wr || rr;
    }
    if (alias) atomicOr(p.err, kRowAlias);
}

}  // namespace

hipError_t launch_align_plan(const PlanParams& p, hipStream_t s)
{
    PlanParams args = p;
    void* kargs[] = {&args};
    const unsigned grid = (unsigned)((p.num_rows + kThreads - 1) / kThreads);
    return hipLaunchKernel(reinterpret_cast<const void*>(&align_plan_kernel), dim3(grid),
                           dim3(kThreads), kargs, 0, s);
}

}  // namespace gdn

#include "gdn_replay.h"

extern "C" int32_t gdn_check_slots(int32_t num_rows, const int32_t* src_slot,
                                   const int32_t* dst_slot, const int32_t* rec_slot,
                                   const int32_t* n_accept, const int32_t* bnd_len,
                                   const int32_t* bnd_slot, int32_t* err_flags, void* stream)
{
    using namespace gdn;
    if (num_rows < 0) return GDN_ERR_SHAPE;
    if (!src_slot || !dst_slot || !n_accept || !err_flags) return GDN_ERR_NULL;
    if ((bnd_len == nullptr) != (bnd_slot == nullptr)) return GDN_ERR_NULL;
    if (num_rows == 0) return GDN_OK;
    SlotCheckParams p{src_slot, dst_slot, rec_slot, n_accept, bnd_len, bnd_slot, err_flags, num_rows};
    void* kargs[] = {&p};
    const unsigned grid = (unsigned)((num_rows + kThreads - 1) / kThreads);
    return hipLaunchKernel(reinterpret_cast<const void*>(&slot_check_kernel), dim3(grid),
                           dim3(kThreads), kargs, 0, (hipStream_t)stream) == hipSuccess
               ? GDN_OK
               : GDN_ERR_LAUNCH;
}
