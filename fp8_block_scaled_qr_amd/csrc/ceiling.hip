// Streaming-read yardstick for the benchmark (not part of the qr ABI; built into its own
// library, libqr_ceiling.so).  One launch reads `bytes` contiguous bytes once: workgroup b of
// `grid` takes the b-th contiguous share, each lane loads 16 bytes per access with four
// accesses in flight, and folds what it read into one word so the loads cannot be dropped.
// Timing it over a buffer the size of a kernel's algorithmic bytes gives the rate a single
// launch of that size can stream on this GPU, against which a bandwidth-bound kernel of the
// same size is judged.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void k_stream_read(const uint4 *__restrict__ p, int64_t n16,
                                                     uint32_t *__restrict__ sink)
{
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
    uint32_t acc = 0;
    int64_t i = b0 + threadIdx.x;
    for (; i + 3 * 256 < b1; i += 4 * 256) {
        const uint4 a = p[i], b = p[i + 256], c = p[i + 512], d = p[i + 768];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
               d.z ^ d.w;
    }
    for (; i < b1; i += 256) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    // one word per workgroup: lane 0 of wave 0 stores the fold of the workgroup's first wave
    // (the other waves' loads are kept by the data dependence of this conditional store)
    acc ^= __shfl_xor(acc, 1) ^ __shfl_xor(acc, 2);
    if (acc == 0x9E3779B9u)
        sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" int qr_ceiling_stream_read(const void *p, int64_t bytes, int32_t grid, void *sink,
                                      void *stream)
{
    if (!p || !sink || bytes < 16 || bytes % 16 != 0 || grid < 1 || grid > 65535 ||
        (reinterpret_cast<uintptr_t>(p) & 15) != 0)
        return 1;
    k_stream_read<<<grid, 256, 0, (hipStream_t)stream>>>(static_cast<const uint4 *>(p), bytes / 16,
                                                         static_cast<uint32_t *>(sink));
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
