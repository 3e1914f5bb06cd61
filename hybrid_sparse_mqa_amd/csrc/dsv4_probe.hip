// dsv4_probe.hip -- a plain streaming read, as a yardstick for the kernels:
// how long this device takes to read a given number of bytes from HBM with
// nothing else to do (no metadata to resolve first, no arithmetic, no
// stores).  Timing only; it computes nothing of the attention.
//
// Workgroup g of G reads bytes [g * share, (g + 1) * share) (share = the
// 16-byte units rounded up over G, the last share shorter), 256 lanes with
// eight 16-byte non-temporal loads each in flight per step.  The loaded
// words are folded into one value per lane, which is stored only if it
// equals a constant no fill of this buffer by the caller is expected to
// produce, so that the compiler keeps the loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsv4_probe.h"

namespace dsv4 {
namespace {

typedef uint32_t pr_u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(256) void read_probe_kernel(const pr_u32x4* __restrict__ buf, int64_t units,
                                                         int64_t share, pr_u32x4* sink) {
    const int64_t lo = (int64_t)blockIdx.x * share;
    const int64_t hi = min(lo + share, units);
    pr_u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t i = lo + threadIdx.x; i < hi; i += 256 * kProbeUnroll) {
        pr_u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int64_t j = i + 256 * u;
            v[u] = j < hi ? __builtin_nontemporal_load(buf + j) : pr_u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
    }
    if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u && acc[2] == 0xf39cc060u && acc[3] == 0x5cedc834u) *sink = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, int64_t bytes, int32_t workgroups, void* sink, hipStream_t stream) {
    const int64_t units = bytes / 16;
    if (units == 0) return hipSuccess;
    const int64_t share = (units + workgroups - 1) / workgroups;
    const unsigned grid = (unsigned)((units + share - 1) / share);  // every workgroup has a nonempty share
    hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, stream, (const pr_u32x4*)buf, units, share,
                       (pr_u32x4*)sink);
    return hipGetLastError();
}

}  // namespace dsv4
