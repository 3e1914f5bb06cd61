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

// Whether a quotient q computed as x * rcp(scale) (within 2 ulp of the
// correctly rounded x / scale) could round to a different E4M3 code than the
// exact quotient: only if it lies within a few ulp of a rounding boundary,
// i.e. of a midpoint between neighbouring codes.  Below 2^-6 the codes are
// the multiples of 2^-9 (midpoints at odd multiples of 2^-10); above, a
// midpoint has exactly the top bit set in the 20 mantissa bits that rounding
// to 3 bits drops (464, the saturation threshold, is one of them).
__device__ __forceinline__ bool near_midpoint(float q) {
    const float a = __builtin_fabsf(q);
    if (a < 0.015625f) {
        const float t = a * 512.0f;  // exact
        return __builtin_fabsf(t - __builtin_floorf(t) - 0.5f) < 1e-5f;
    }
    return ((__builtin_bit_cast(uint32_t, a) & 0xFFFFFu) - 0x7FFF8u) <= 16u;  // within 8 of 0x80000
}

// Four floats -> four OCP E4M3FN codes (bytes 0..3 in order) with gfx950's
// conversion instruction (round to nearest even), after clamping to +-448 so
// that larger magnitudes saturate (clamping keeps the sign of zeros).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    auto clamp = [](float x) { return __builtin_fminf(__builtin_fmaxf(x, -448.0f), 448.0f); };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(a), clamp(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(c), clamp(d), w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// This lane's share of a row's largest non-rotary magnitude (lane l holds
// dims 8l .. 8l+7 in v: lanes 0..55 the non-rotary part, 56..63 the rotary).
__device__ __forceinline__ float lane_amax(const pk_u32x4& v, int l) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(__builtin_fabsf(bf16_lo(v[j])), __builtin_fabsf(bf16_hi(v[j]))));
    return l < 56 ? amax : 0.f;
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
        // The quotients by a reciprocal multiply; where one of the wave's
        // could round differently from the correctly rounded quotient (or the
        // scale is subnormal, where the reciprocal overflows), by division.
        const float r = __builtin_amdgcn_rcpf(scale);
        float q[8];
        bool risky = false;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            q[j] = f[j] * r;
            risky |= near_midpoint(q[j]);
        }
        if (__builtin_expect(__any(risky) || !(scale >= 1.17549435e-38f), 0)) {
#pragma unroll
            for (int j = 0; j < 8; ++j) q[j] = f[j] / scale;
        }
        *(pk_u32x2*)(rec + 8 * l) = pk_u32x2{e4m3x4(q[0], q[1], q[2], q[3]), e4m3x4(q[4], q[5], q[6], q[7])};
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
    // The rows' maxima over the wave, their shuffles interleaved.
    float amax[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) amax[r] = lane_amax(v[r], l);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) amax[r] = fmaxf(amax[r], __shfl_xor(amax[r], o));
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
        if (slot[r] >= 0) pack_row(p, v[r], slot[r], amax[r], l);
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
