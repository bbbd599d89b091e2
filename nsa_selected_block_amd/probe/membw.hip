// membw.hip -- read-bandwidth probe used by the benchmark (bench.py --branch
// membw): how fast the GPU streams a working set of a given size, so that
// the memory-side cache (256 MB on MI355X) can be told apart from HBM.
// Built as its own library, libnsa_probe.so; the selected-attention library
// does not contain or call it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

// Every thread reads 16-byte words of [base, base + bytes) with a grid
// stride, `reps` passes over the buffer, and folds them into one word per
// thread (stored, so the loads stay).  Four independent loads per thread are
// in flight per step; they use the default cache policy, as the library's
// kernels do.
__global__ __launch_bounds__(256) void k_read(const uint4* __restrict__ base, uint64_t n16, int reps,
                                              uint32_t* __restrict__ sink)
{
    const uint64_t tid = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    uint32_t acc = 0;
    for (int r = 0; r < reps; ++r) {
        uint64_t i = tid;
        for (; i + 3 * stride < n16; i += 4 * stride) {
            const uint4 a = base[i];
            const uint4 b = base[i + stride];
            const uint4 c = base[i + 2 * stride];
            const uint4 d = base[i + 3 * stride];
            acc ^= a.x ^ a.w ^ b.y ^ b.z ^ c.x ^ c.w ^ d.y ^ d.z;
        }
        for (; i < n16; i += stride) {
            const uint4 a = base[i];
            acc ^= a.x ^ a.w;
        }
    }
    sink[tid] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) at `buf` `reps` times on `stream` with
// `blocks` workgroups of 256 threads; `sink` takes blocks * 256 words.
// Returns 0, or the HIP error code of the launch.
int nsa_probe_read(const void* buf, uint64_t bytes, int reps, int blocks, uint32_t* sink, void* stream)
{
    if (!buf || !sink || bytes % 16 || reps < 1 || blocks < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_read, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4*>(buf), bytes / 16, reps, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
