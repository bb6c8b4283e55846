// Measurement aid, not part of the matmul path: a plain streaming read of a
// device buffer, used to measure the bandwidth a kernel that only reads HBM
// reaches at a given byte count (the practical ceiling the matmul is
// compared against).  Built into its own library, libw4a16_probe.so.
//
// Each workgroup reads one contiguous chunk with 16-byte non-temporal loads,
// U independent loads in flight per thread; the words are XOR-folded and the
// fold is stored only when it hits an unlikely value, so the loads cannot be
// removed and almost nothing is written.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ void __launch_bounds__(1024) stream_read(const u32x4 *__restrict__ src, long long n16,
                                                    long long chunk16, uint32_t *__restrict__ sink) {
    const long long begin = (long long)blockIdx.x * chunk16;
    const long long end = begin + chunk16 < n16 ? begin + chunk16 : n16;
    uint32_t fold = 0;
    for (long long i = begin + threadIdx.x; i < end; i += (long long)blockDim.x * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long long j = i + (long long)u * blockDim.x;
            v[u] = j < end ? __builtin_nontemporal_load(src + j) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) fold ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (fold == 0x9E3779B9u) sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = fold;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from `src` with `blocks` x `threads`
// threads and `unroll` loads in flight per thread (1, 4 or 8).  `sink` must
// hold blocks * threads uint32 values.  Returns 0, or -1 for bad arguments,
// -2 if the launch failed.
extern "C" int w4a16_probe_stream_read(const void *src, long long bytes, int blocks, int threads,
                                       int unroll, void *sink, void *stream) {
    if (!src || !sink || bytes <= 0 || bytes % 16 || blocks <= 0 || threads <= 0 || threads > 1024 ||
        threads % 64)
        return -1;
    const long long n16 = bytes / 16;
    const long long chunk16 = (n16 + blocks - 1) / blocks;
    const u32x4 *s = static_cast<const u32x4 *>(src);
    uint32_t *o = static_cast<uint32_t *>(sink);
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (unroll) {
    case 1: hipLaunchKernelGGL(stream_read<1>, dim3(blocks), dim3(threads), 0, st, s, n16, chunk16, o); break;
    case 4: hipLaunchKernelGGL(stream_read<4>, dim3(blocks), dim3(threads), 0, st, s, n16, chunk16, o); break;
    case 8: hipLaunchKernelGGL(stream_read<8>, dim3(blocks), dim3(threads), 0, st, s, n16, chunk16, o); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}
