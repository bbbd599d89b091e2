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

// Gathers of 1 KB pieces (one 16-byte load per lane of a wave) at
// pseudo-random piece indices of [base, base + 1 KB * npieces): each wave
// issues K loads, then folds them, `iters` times.  The loads are
// non-temporal, as the merges' partial reads are.  The piece index is a
// 32-bit mix (multiply, xor-shift) of (wave, iteration, load), uniform over
// the wave.
template <int K>
__global__ __launch_bounds__(256) void k_gather(const uint4* __restrict__ base, uint32_t npieces, int iters,
                                                uint32_t* __restrict__ sink)
{
    const uint32_t wave = (blockIdx.x * 256 + threadIdx.x) >> 6, lane = threadIdx.x & 63;
    uint32_t acc = 0;
    for (int it = 0; it < iters; ++it) {
        uint4 v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            uint32_t h = (wave * 0x9E3779B1u) ^ ((uint32_t)it * 0x85EBCA77u) ^ ((uint32_t)k * 0xC2B2AE3Du);
            h ^= h >> 15;
            h *= 0x2C1B3C6Du;
            h ^= h >> 13;
            const uint64_t i = (uint64_t)(h % npieces) * 64 + lane;
            const uint32_t* w = reinterpret_cast<const uint32_t*>(base + i);
            v[k] = make_uint4(__builtin_nontemporal_load(w), __builtin_nontemporal_load(w + 1),
                              __builtin_nontemporal_load(w + 2), __builtin_nontemporal_load(w + 3));
        }
#pragma unroll
        for (int k = 0; k < K; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    sink[blockIdx.x * 256 + threadIdx.x] = acc;
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

// Gathers `iters` x 13 pieces of 1 KB per wave from the first `bytes` (a
// multiple of 1024) at `buf`, on `stream` with `blocks` workgroups of 256
// threads (13 loads in flight per wave, as in the merges); `sink` takes
// blocks * 256 words.  Returns 0, or the HIP error code of the launch.
int nsa_probe_gather(const void* buf, uint64_t bytes, int iters, int blocks, uint32_t* sink, void* stream)
{
    if (!buf || !sink || bytes % 1024 || bytes / 1024 == 0 || bytes / 1024 > 0xFFFFFFFFull || iters < 1 ||
        blocks < 1)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_gather<13>, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4*>(buf), (uint32_t)(bytes / 1024), iters, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
