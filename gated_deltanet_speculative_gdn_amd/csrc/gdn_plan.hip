// gdn_plan.hip -- align-mode commit plan, one thread per row, for gfx950.
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
