// HBM read-bandwidth calibration for the benchmark (libmoe_calib.so; not a
// step of the layer and not part of include/moe.h): every 16-byte word of a
// device buffer is read once with the non-temporal hint, eight loads in flight
// per lane, each workgroup streaming one contiguous share of the buffer.  The
// XOR of the words is written per thread so that no load is optimised away.
// The bandwidth it reaches is the attainable read ceiling that the HBM-bound
// grouped GEMMs are compared with.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 1024;
constexpr int kInFlight = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ p, uint64_t n16,
                                                              unsigned* __restrict__ out)
{
    const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const uint64_t beg = (uint64_t)blockIdx.x * per;
    const uint64_t end = beg + per < n16 ? beg + per : n16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    uint64_t i = beg + threadIdx.x;
    for (; i + (uint64_t)(kInFlight - 1) * kThreads < end; i += (uint64_t)kInFlight * kThreads) {
        u32x4 v[kInFlight];
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) v[j] = __builtin_nontemporal_load(p + i + (uint64_t)j * kThreads);
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) acc ^= v[j];
    }
    for (; i < end; i += kThreads) acc ^= __builtin_nontemporal_load(p + i);
    out[(uint64_t)blockIdx.x * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) at device pointer `buf` once; `out` is a
// device buffer of grid * 1024 unsigned ints; `grid` workgroups of 1024
// threads.  Asynchronous on `stream`; returns 0 or a hipError_t value.
int moe_calib_stream_read(const void* buf, uint64_t bytes, unsigned* out, int grid, void* stream)
{
    if (!buf || !out || grid < 1 || bytes % 16) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), bytes / 16, out);
    return (int)hipGetLastError();
}

}  // extern "C"
