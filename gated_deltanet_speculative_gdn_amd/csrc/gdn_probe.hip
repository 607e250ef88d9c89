// gdn_probe.hip -- HBM bandwidth probe (read, write, copy) for gfx950, and its
// C ABI (include/gdn_probe.h).
//
// A measurement aid beside the replay kernels: each workgroup of four wave64s
// streams one 16 KiB chunk with 16-byte non-temporal accesses, thread t taking
// pieces t + 256 i (i < 4), so that each load or store instruction of the
// workgroup covers 4 KiB of contiguous memory -- the all-layer commit's state
// access pattern -- and workgroup ids are remapped XCD-contiguous as in the
// commit. The read kernel folds its chunk into one 16-byte XOR word (a lane
// XOR over each wave, then over the four waves through LDS) so that no load
// can be dropped, and writes that word: 1/1024 of the bytes read.
#include <hip/hip_runtime.h>

#include "gdn_device.hpp"
#include "gdn_probe.h"
#include "gdn_replay.h"

namespace gdn {
namespace {

constexpr int kProbePer = GDN_PROBE_CHUNK / 16 / kThreads;   // 16-byte pieces per thread
static_assert(kProbePer * 16 * kThreads == GDN_PROBE_CHUNK, "chunk = 256 threads x pieces");

__device__ __forceinline__ u32x4 xor_lanes(u32x4 x)
{
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        x.x ^= (uint32_t)__shfl_xor((int)x.x, m);
        x.y ^= (uint32_t)__shfl_xor((int)x.y, m);
        x.z ^= (uint32_t)__shfl_xor((int)x.z, m);
        x.w ^= (uint32_t)__shfl_xor((int)x.w, m);
    }
    return x;
}

template <int KIND>
__global__ void __launch_bounds__(kThreads) probe_kernel(const u32x4* src, u32x4* dst)
{
    const int64_t chunk = xcd_contiguous_id(blockIdx.x, gridDim.x);
    const int64_t base = chunk * (GDN_PROBE_CHUNK / 16);
    const int t = threadIdx.x;
    if constexpr (KIND == GDN_PROBE_WRITE) {
        const uint32_t v = (uint32_t)chunk;
#pragma unroll
        for (int i = 0; i < kProbePer; ++i)
            __builtin_nontemporal_store(u32x4{v, v, v, v}, dst + base + t + kThreads * i);
    } else {
        u32x4 x[kProbePer];
#pragma unroll
        for (int i = 0; i < kProbePer; ++i)
            x[i] = __builtin_nontemporal_load(src + base + t + kThreads * i);
        if constexpr (KIND == GDN_PROBE_COPY) {
#pragma unroll
            for (int i = 0; i < kProbePer; ++i)
                __builtin_nontemporal_store(x[i], dst + base + t + kThreads * i);
        } else {
            u32x4 acc = x[0];
#pragma unroll
            for (int i = 1; i < kProbePer; ++i) acc ^= x[i];
            acc = xor_lanes(acc);
            __shared__ u32x4 wave_acc[kThreads / 64];
            if ((t & 63) == 0) wave_acc[t >> 6] = acc;
            __syncthreads();
            if (t == 0) {
                u32x4 r = wave_acc[0];
#pragma unroll
                for (int w = 1; w < kThreads / 64; ++w) r ^= wave_acc[w];
                dst[chunk] = r;
            }
        }
    }
}

}  // namespace
}  // namespace gdn

extern "C" int32_t gdn_bandwidth_probe(int32_t kind, const void* src, void* dst, int64_t bytes,
                                       void* stream)
{
    using namespace gdn;
    if (kind != GDN_PROBE_READ && kind != GDN_PROBE_WRITE && kind != GDN_PROBE_COPY)
        return GDN_ERR_SHAPE;
    if (bytes <= 0 || bytes % GDN_PROBE_CHUNK != 0 || bytes / GDN_PROBE_CHUNK > INT32_MAX)
        return GDN_ERR_SHAPE;
    if (!dst || (kind != GDN_PROBE_WRITE && !src)) return GDN_ERR_NULL;
    if (((uintptr_t)dst & 15u) || (kind != GDN_PROBE_WRITE && ((uintptr_t)src & 15u)))
        return GDN_ERR_ALIGN;
    const dim3 grid((unsigned)(bytes / GDN_PROBE_CHUNK));
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    void* args[] = {&s, &d};
    const void* fn = kind == GDN_PROBE_READ    ? reinterpret_cast<const void*>(&probe_kernel<GDN_PROBE_READ>)
                     : kind == GDN_PROBE_WRITE ? reinterpret_cast<const void*>(&probe_kernel<GDN_PROBE_WRITE>)
                                               : reinterpret_cast<const void*>(&probe_kernel<GDN_PROBE_COPY>);
    return hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, (hipStream_t)stream) == hipSuccess
               ? GDN_OK
               : GDN_ERR_LAUNCH;
}
