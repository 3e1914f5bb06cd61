// dsv4_pack.hip -- the KV store on the decode path: new K rows quantised into
// packed FP8 records (the cache write of "DeepSeek-V4 Attention: Query, cache
// write and history addressing", section 3 (k = v); the 584-byte record of
// FP8 non-rotary dims + bf16 rotary dims of the "SGLang DeepSeek-V4 attention
// test capability matrix" page).  Record layout inside a page: the library's
// (include/dsv4_attn.h): 256 records of 576 bytes [448 E4M3FN codes | 64 bf16
// rotary dims], then 256 fp32 per-token scales.
//
// Per row: scale = max |nope| / 448 in float (1 if every non-rotary dim is
// zero); code = E4M3FN(nope / scale) with the division in float, rounded to
// the nearest finite value, ties to the even code, large magnitudes
// saturating to 448; the rotary dims are copied.  HBM-bound: 1 KiB read and
// 580 bytes written per row, one wave per row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsv4_launch.h"

namespace dsv4 {
namespace {

typedef uint32_t pk_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t pk_u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRecBytes = 576;
constexpr int kScaleOffset = 256 * kRecBytes;

// float -> OCP E4M3FN code, round to nearest even, saturating at 448; the
// sign bit of x becomes the code's (x finite).  Below 2^-6 the codes are the
// multiples of 2^-9 (subnormals, and 8 -> the smallest normal 2^-6), so the
// magnitude is rounded to an integer count of 2^-9; above, the float's 23
// mantissa bits are rounded to 3 (a carry moves into the exponent).
__device__ __forceinline__ uint32_t e4m3_code(float x) {
    const uint32_t bits = __builtin_bit_cast(uint32_t, x);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const float a = __builtin_fabsf(x);
    uint32_t mag;
    if (!(a < 464.0f)) {  // 464 is the midpoint between 448 and the (non-finite) next step
        mag = 0x7Eu;
    } else if (a < 0.015625f) {
        mag = (uint32_t)__builtin_rintf(a * 512.0f);  // exact scaling; rint rounds half to even
    } else {
        uint32_t ab = bits & 0x7FFFFFFFu;
        ab += 0x7FFFFu + ((ab >> 20) & 1u);
        mag = min((((ab >> 23) - 120u) << 3) | ((ab >> 20) & 7u), 0x7Eu);
    }
    return sign | mag;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Wave w of a workgroup packs row 4*blockIdx.x + w; lane l holds dims
// 8l .. 8l+7 (lanes 0..55 the non-rotary part, 56..63 the rotary part).
__global__ __launch_bounds__(256) void pack_fp8_kernel(PackArgs p) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int l = threadIdx.x & 63;
    if (row >= p.n) return;
    const int32_t slot = p.slots[row];  // uniform over the wave
    if (slot < 0) return;
    const pk_u32x4 v = *(const pk_u32x4*)(p.k + row * p.k_s0 + 8 * l);
    float f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = bf16_lo(v[j]);
        f[2 * j + 1] = bf16_hi(v[j]);
    }
    float amax = 0.f;
    if (l < 56) {
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, __builtin_fabsf(f[j]));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    uint8_t* page = p.pool + (int64_t)(slot >> 8) * p.page_bytes;
    uint8_t* rec = page + (slot & 255) * kRecBytes;
    if (l < 56) {
        uint32_t c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = e4m3_code(f[j] / scale);
        *(pk_u32x2*)(rec + 8 * l) = pk_u32x2{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                                             c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
    } else {
        *(pk_u32x4*)(rec + 448 + 16 * (l - 56)) = v;
    }
    if (l == 0) *(float*)(page + kScaleOffset + 4 * (slot & 255)) = scale;
}

}  // namespace

hipError_t launch_pack_fp8(const PackArgs& p, hipStream_t stream) {
    if (p.n == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_fp8_kernel, dim3((unsigned)((p.n + 3) / 4)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace dsv4
