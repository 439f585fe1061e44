// gdn_common.h -- small device helpers used by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// bf16 <-> fp32.  bf16 is the top half of an fp32 bit pattern.
__device__ __forceinline__ float bf16_to_f32(uint16_t b)
{
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even.  Inputs are finite in this library; NaN is
// kept a NaN by forcing a mantissa bit.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Sum over each aligned group of 32 lanes of a wave64; every lane of the group
// receives the total.  Four DPP steps reduce within rows of 16 lanes (swap
// neighbours, swap pairs, mirror within 8, mirror within 16); one ds_swizzle
// (xor 16, bit mode) folds the two rows of the 32-lane group.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL,
                                                      0xf, 0xf, false));
}

__device__ __forceinline__ float sum32(float x)
{
    x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);  // row_half_mirror
    x += dpp_mov<0x140>(x);  // row_mirror
    x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
    return x;
}

// ---- LDS-DMA helpers ----------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void global_cvoid;

// One 16-byte-per-lane LDS-DMA: lane l's 16 bytes (from base + off) land at
// lds + 16 l.  base and lds are wave-uniform; off is a per-lane byte offset.
__device__ __forceinline__ void dma16(const unsigned char *base, uint32_t off, void *lds)
{
    __builtin_amdgcn_global_load_lds((global_cvoid *)(base + off), (lds_void *)(lds), 16, 0, 0);
}

// Wait until at most N of this wave's global loads (LDS-DMA included) are
// outstanding; they complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vmem_le()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // s_waitcnt fields: vmcnt[3:0], expcnt[6:4] (7 = no wait), lgkmcnt[11:8]
    // (15 = no wait), vmcnt[5:4] in bits 15:14
    __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14));
}

// Byte offset, inside one chunk's data, of the 16 bytes lane `lane` loads for LDS
// block `blk` of a padded region: rows of `rowb` valid bytes stored with stride
// `stride`; pad slots read offset 0.  `gstride` is the source row stride; rows at
// or past nv read row nv - 1.
__device__ __forceinline__ uint32_t dma_src_offset(int blk, int lane, int rowb, int stride,
                                                   uint32_t gstride, int nv)
{
    const int o = blk * 1024 + lane * 16;
    const int r = o / stride, b = o - r * stride;
    const uint32_t v = uint32_t(min(r, nv - 1)) * gstride + uint32_t(b);
    return b < rowb ? v : 0u;
}

// Input transforms applied inside the op on request (fp32).
// Epsilon inside the root of the q/k row normalisation: an all-zero row stays zero.
constexpr float kL2Eps = 1e-6f;

// g := -softplus(x) = -log(1 + e^x), written as -(max(x, 0) + log1p(e^-|x|)) so
// that neither branch overflows.
__device__ __forceinline__ float neg_softplus(float x)
{
    return -(fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))));
}

// beta := sigmoid(x) = 1 / (1 + e^-x)
__device__ __forceinline__ float sigmoid(float x)
{
    return 1.f / (1.f + expf(-x));
}

}  // namespace gdn
