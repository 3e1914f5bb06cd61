// dsv4_probe.h -- launcher of the plain streaming-read timing kernel
// (dsv4_probe.hip); kept apart from the attention kernels' launch header.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsv4 {
hipError_t launch_read_probe(const void* buf, int64_t bytes, int32_t workgroups, void* sink, hipStream_t stream);
}  // namespace dsv4
