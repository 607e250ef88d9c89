// gdn_device.hpp -- device helpers for the gfx950 verify / commit kernels.
//
// Wave64 on CDNA4: reductions over 8 or 16 consecutive lanes use DPP lane
// permutes inside one 16-lane DPP row (quad permutes, then the half-row and
// row mirrors), never LDS. Each step adds a lane's value to its partner's;
// IEEE addition is commutative, so after every step all lanes of the group
// hold the bit-identical sum. Every kernel built from these helpers is
// compiled with floating-point contraction off: an fma is issued only where
// the method fuses one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kDim = 128;          // K = V = 128
constexpr int kHeadElems = kDim * kDim;
constexpr int kThreads = 256;      // four wave64s per workgroup
constexpr float kNormEps = 1e-6f;  // inside the square root of the L2 norm
constexpr float kSoftplusLinear = 20.f;  // softplus(x) = x above this input

// Row-error bits, the values the C ABI documents.
constexpr int kRowSlot = 1, kRowWin = 2, kRowN = 4, kRowBnd = 8, kRowTable = 16,
              kRowRec = 32, kRowPos = 64, kRowAlias = 128;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- bf16 ------------------------------------------------------------------
// A bf16 value is the top half of an fp32 value: widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

// Two values rounded to bf16, nearest with ties to even, packed (lo in the
// low half): gfx950's conversion instruction, one per pair. It rounds fp32
// subnormals too (they are kept: no flush-to-zero here) and gives a quiet NaN
// for a NaN; a GPU test holds it to an integer round-to-nearest-even over the
// whole fp32 range.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// ---- DPP lane exchange -----------------------------------------------------
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7-i inside each 8 lanes
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15-i inside each 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 8 lanes 8m..8m+7; every one of them returns the same bits.
__device__ __forceinline__ float sum8(float x) {
    x = x + dpp<kDppQuadXor1>(x);
    x = x + dpp<kDppQuadXor2>(x);
    x = x + dpp<kDppRowHalfMirror>(x);
    return x;
}

// Sum over the 16 lanes of a DPP row.
__device__ __forceinline__ float sum16(float x) {
    x = sum8(x);
    return x + dpp<kDppRowMirror>(x);
}

// Sum over the 32 lanes 32m..32m+31: the 16-lane sums of the two DPP rows,
// then one swap of the halves (ds_swizzle, xor 16 within 32 lanes).
__device__ __forceinline__ float sum32(float x) {
    x = sum16(x);
    constexpr int kSwizzleXor16 = 0x401F;    // bit mode: and 0x1f, or 0, xor 0x10
    return x + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), kSwizzleXor16));
}

// L2 normalisation of a 128-vector held as 8 consecutive elements per lane
// across the 16 lanes of a DPP row: x * (1 / sqrt(sum x^2 + eps)), the sum
// taken as 8 fmas in the lane and a 16-lane DPP sum. Every kernel that needs a
// normalised key calls this, so they all produce the same bits.
__device__ __forceinline__ void l2norm_row16(float (&x)[8]) {
    float ssq = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ssq = __builtin_fmaf(x[i], x[i], ssq);
    ssq = sum16(ssq);
    const float inv = 1.0f / __builtin_sqrtf(ssq + kNormEps);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = x[i] * inv;
}

// ---- vector memory ---------------------------------------------------------
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void st4_nt(float* p, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ f32x4 ld4_nt(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}

// Uniform read of a kernel input the kernel never writes (row metadata):
// through the constant address space with a wave-uniform index it becomes a
// scalar load, which waits on its own counter rather than on the vector loads
// in flight.
__device__ __forceinline__ int32_t ld_uniform(const int32_t* base, int idx) {
    typedef const __attribute__((address_space(4))) int32_t cint32;
    const int i = __builtin_amdgcn_readfirstlane(idx);
    return ((cint32*)base)[i];
}

// The dispatcher hands workgroup w to XCD w % 8 (eight XCDs, each with its
// own L2). Remapping w so that the workgroups one XCD receives take one
// contiguous range of logical ids lets each XCD stream a contiguous stretch of
// memory instead of every eighth piece. A bijection on [0, grid); the tail
// past the last multiple of 8 keeps its id.
constexpr int kNumXcd = 8;
__device__ __forceinline__ uint32_t xcd_contiguous_id(uint32_t w, uint32_t grid) {
    const uint32_t per = grid / kNumXcd;
    return w < per * kNumXcd ? (w % kNumXcd) * per + w / kNumXcd : w;
}

}  // namespace gdn
