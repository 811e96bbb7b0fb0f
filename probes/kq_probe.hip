// kq_probe.hip -- the roofline probes of kq_probe.h: a plain streaming read
// and a plain int8 matrix-core loop, each the simplest kernel of its kind,
// so the matmul kernels' fractions can be quoted against what this
// hardware reaches as well as against the datasheet.
#include "kq.h"
#include "kq_probe.h"

#include <hip/hip_runtime.h>

namespace kq {
namespace {

// Streaming read with U 16-byte loads in flight per thread: each thread
// reads words i, i + nth, ..., i + (U-1)*nth of a block of U*nth words, then
// the grid strides to the next block.
template <int U>
__global__ __launch_bounds__(256) void probe_read_kernel(const uint4 *__restrict__ p, int64_t words,
                                                         uint32_t *__restrict__ sink)
{
    const int64_t nth = (int64_t)gridDim.x * 256;
    uint32_t acc = 0;
    for (int64_t base = (int64_t)blockIdx.x * 256 + threadIdx.x; base < words; base += nth * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * nth;
            v[u] = i < words ? p[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void probe_mfma_kernel(int64_t iters, int32_t *__restrict__ sink)
{
    const int l = threadIdx.x & 63;
    const i32x4 a = {l, 3 * l, 5, 7}, b = {7 * l, l, 3, 1};
    i32x16 acc[4] = {};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[j], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[j][0] ^ acc[j][15];
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace
}  // namespace kq

extern "C" {

int kq_probe_read_u(const void *buf, size_t bytes, uint32_t *sink, int grid, int unroll, void *stream)
{
    if (!buf || !sink || bytes == 0 || bytes % 16 || grid < 1 || grid > 65536) return KQ_EINVAL;
    if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8 && unroll != 16) return KQ_EINVAL;
    if ((uintptr_t)buf % 16 || (uintptr_t)sink % 4) return KQ_EALIGN;
    const uint4 *p = (const uint4 *)buf;
    const int64_t words = (int64_t)(bytes / 16);
    const hipStream_t st = (hipStream_t)stream;
    switch (unroll) {
    case 1: hipLaunchKernelGGL(kq::probe_read_kernel<1>, dim3((unsigned)grid), dim3(256), 0, st, p, words, sink); break;
    case 2: hipLaunchKernelGGL(kq::probe_read_kernel<2>, dim3((unsigned)grid), dim3(256), 0, st, p, words, sink); break;
    case 4: hipLaunchKernelGGL(kq::probe_read_kernel<4>, dim3((unsigned)grid), dim3(256), 0, st, p, words, sink); break;
    case 8: hipLaunchKernelGGL(kq::probe_read_kernel<8>, dim3((unsigned)grid), dim3(256), 0, st, p, words, sink); break;
    default: hipLaunchKernelGGL(kq::probe_read_kernel<16>, dim3((unsigned)grid), dim3(256), 0, st, p, words, sink);
    }
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ELAUNCH;
}

int kq_probe_read(const void *buf, size_t bytes, uint32_t *sink, int grid, void *stream)
{
    return kq_probe_read_u(buf, bytes, sink, grid, 4, stream);
}

int kq_probe_mfma_i8(int64_t iters, int grid, int32_t *sink, void *stream)
{
    if (!sink || iters < 1 || iters > ((int64_t)1 << 24) || grid < 1 || grid > 65536) return KQ_EINVAL;
    if ((uintptr_t)sink % 4) return KQ_EALIGN;
    hipLaunchKernelGGL(kq::probe_mfma_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, iters, sink);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ELAUNCH;
}

}  // extern "C"
