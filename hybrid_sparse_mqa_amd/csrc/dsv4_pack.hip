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
// saturating to 448; the rotary dims are copied.  1 KiB read and 580 bytes
// written per row, one wave per row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsv4_launch.h"

namespace dsv4 {
namespace {

typedef uint32_t pk_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t pk_u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRecBytes = 576;
constexpr int kScaleOffset = 256 * kRecBytes;

// Four floats -> four OCP E4M3FN codes (bytes 0..3 in order) with gfx950's
// conversion instruction (round to nearest even).  kClamp: clamp to +-448
// first, so that larger magnitudes saturate (clamping keeps the sign of
// zeros); callers whose values cannot exceed 448 by more than a rounding
// error skip it (such values still round to 448).
template <bool kClamp>
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    auto clamp = [](float x) { return kClamp ? __builtin_fminf(__builtin_fmaxf(x, -448.0f), 448.0f) : x; };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(a), clamp(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(c), clamp(d), w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// This lane's share of a row's largest non-rotary magnitude, as bf16 bits
// (lane l holds dims 8l .. 8l+7 in v: lanes 0..55 the non-rotary part,
// 56..63 the rotary).  Finite bf16 magnitudes order like their bit patterns
// with the sign cleared, so the maximum is taken on those, two per packed
// 16-bit integer max.
typedef uint16_t pk_u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t lane_amax_bits(const pk_u32x4& v, int l) {
    pk_u16x2 m = __builtin_bit_cast(pk_u16x2, v[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int j = 1; j < 4; ++j) m = __builtin_elementwise_max(m, __builtin_bit_cast(pk_u16x2, v[j] & 0x7FFF7FFFu));
    const uint32_t r = max((uint32_t)m[0], (uint32_t)m[1]);
    return l < 56 ? r : 0u;
}

// One row, given its largest non-rotary magnitude.
__device__ __forceinline__ void pack_row(const PackArgs& p, const pk_u32x4& v, int32_t slot, float amax, int l) {
    float f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = bf16_lo(v[j]);
        f[2 * j + 1] = bf16_hi(v[j]);
    }
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    uint8_t* page = p.pool + (int64_t)(slot >> 8) * p.page_bytes;
    uint8_t* rec = page + (slot & 255) * kRecBytes;
    if (l < 56) {
        // The codes of the correctly rounded quotients f / scale, without a
        // division: q = f * rcp(scale) lies within 2 ulp of the correctly
        // rounded quotient (rcp is within 1 ulp), so that quotient lies
        // between q (1 - 2^-21) and q (1 + 2^-21), computed here as f * ra
        // and f * rb (each within 1 more ulp).  Rounding to E4M3 is
        // monotone, so where both bounds give the same code, so does the
        // quotient.  Where one of the wave's pairs differs (the quotient is
        // within a few ulp of a rounding midpoint), or the scale is
        // subnormal (its reciprocal overflows), the quotients are divided.
        // |f| <= amax = 448 scale, so no quotient exceeds 448 by more than a
        // rounding error and none needs the saturating clamp.
        const float r = __builtin_amdgcn_rcpf(scale);
        const float ra = r * (1.0f - 0x1p-21f), rb = r * (1.0f + 0x1p-21f);
        uint32_t c0 = e4m3x4<false>(f[0] * ra, f[1] * ra, f[2] * ra, f[3] * ra);
        uint32_t c1 = e4m3x4<false>(f[4] * ra, f[5] * ra, f[6] * ra, f[7] * ra);
        const uint32_t d0 = e4m3x4<false>(f[0] * rb, f[1] * rb, f[2] * rb, f[3] * rb);
        const uint32_t d1 = e4m3x4<false>(f[4] * rb, f[5] * rb, f[6] * rb, f[7] * rb);
        if (__builtin_expect(__any((c0 != d0) | (c1 != d1)) || !(scale >= 1.17549435e-38f), 0)) {
            float q[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) q[j] = f[j] / scale;
            c0 = e4m3x4<true>(q[0], q[1], q[2], q[3]);
            c1 = e4m3x4<true>(q[4], q[5], q[6], q[7]);
        }
        *(pk_u32x2*)(rec + 8 * l) = pk_u32x2{c0, c1};
    } else {
        *(pk_u32x4*)(rec + 448 + 16 * (l - 56)) = v;
    }
    if (l == 0) *(float*)(page + kScaleOffset + 4 * (slot & 255)) = scale;
}

// Wave w of workgroup b packs rows kRowsPerWave * (4b + w) + 0 .. kRowsPerWave-1,
// loading all of them before packing any.  Several rows per wave put more
// bytes in flight per wave (large calls); one row per wave gives the most
// waves and the shortest chain per wave (small calls, e.g. a decode step).
template <int kRowsPerWave>
__global__ __launch_bounds__(256) void pack_fp8_kernel(PackArgs p) {
    const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kRowsPerWave;
    const int l = threadIdx.x & 63;
    if (row0 >= p.n) return;
    pk_u32x4 v[kRowsPerWave];
    int32_t slot[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
        const int64_t row = min(row0 + r, p.n - 1);  // rows past n: a valid address, skipped below
        v[r] = *(const pk_u32x4*)(p.k + row * p.k_s0 + 8 * l);
        slot[r] = row0 + r < p.n ? p.slots[row] : -1;
    }
    // The rows' maxima over the wave (as bf16 bits), their shuffles interleaved.
    uint32_t amax[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) amax[r] = lane_amax_bits(v[r], l);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) amax[r] = max(amax[r], (uint32_t)__shfl_xor((int)amax[r], o));
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
        if (slot[r] >= 0) pack_row(p, v[r], slot[r], __builtin_bit_cast(float, amax[r] << 16), l);
}

}  // namespace

hipError_t launch_pack_fp8(const PackArgs& p, hipStream_t stream) {
    if (p.n == 0) return hipSuccess;
    // Four rows per wave once that still gives every SIMD several waves
    // (measured: 65536 rows 29.4 us with four, 31.5 us with one; 64 rows
    // 2.6 us with one, 5.0 us with four).
    if (p.n >= 16384) {
        hipLaunchKernelGGL(pack_fp8_kernel<4>, dim3((unsigned)((p.n + 15) / 16)), dim3(256), 0, stream, p);
    } else {
        hipLaunchKernelGGL(pack_fp8_kernel<1>, dim3((unsigned)((p.n + 3) / 4)), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace dsv4
