// kq_quantize.hip -- Q8_K activation quantiser (gfx950).
//
// Q8_K form (K-quant kernel arc page, "The pieces", kq v2 item; the k4 v2
// commit message): per 256 activations one float scale d8 = amax/127, int8
// codes a = round(x/d8), and an int16 sum of every 16 codes.  Both divisions
// are correctly rounded binary32 (__fdiv_rn) and the rounding is half to
// even (rintf), so the image is bit-identical to any IEEE implementation of
// the same definition.
//
// One wave per 256-value chunk: each lane owns 4 consecutive values (one
// 16-byte load, one 4-byte store), the chunk's amax is a wave reduction, and
// each 16-value bsum is the sum over a quad of lanes.
#include "kq_common.h"

namespace kq {

__global__ __launch_bounds__(256) void quantize_q8k_kernel(const float *__restrict__ x, int64_t chunks,
                                                           int8_t *__restrict__ xq, float *__restrict__ xs,
                                                           int16_t *__restrict__ xbs)
{
    const int lane = threadIdx.x & 63;
    const int64_t chunk = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (chunk >= chunks) return;  // whole wave exits together

    const float4 v = reinterpret_cast<const float4 *>(x + chunk * QK)[lane];
    int qsum;
    float d8;
    const uint32_t packed = q8k_chunk(v, qsum, d8);
    reinterpret_cast<uint32_t *>(xq + chunk * QK)[lane] = packed;
    // lanes 4g..4g+3 hold the 16 codes of group g
    if ((lane & 3) == 0) xbs[chunk * 16 + (lane >> 2)] = (int16_t)qsum;
    if (lane == 0) xs[chunk] = d8;
}

int launch_quantize_q8k(const float *x, int64_t t, int64_t k, int8_t *xq, float *xs, int16_t *xbs,
                        hipStream_t stream)
{
    const int64_t chunks = t * (k / QK);
    const int per_block = 4;  // waves (chunks) per 256-thread workgroup
    const int64_t blocks = (chunks + per_block - 1) / per_block;
    hipLaunchKernelGGL(quantize_q8k_kernel, dim3((unsigned)blocks), dim3(64 * per_block), 0, stream, x,
                       chunks, xq, xs, xbs);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ELAUNCH;
}

}  // namespace kq
