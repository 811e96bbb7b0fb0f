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
//
// Two code layouts.  The row image is xq[t][k].  The tile image feeds the
// GEMM's MFMA A operand: tokens in groups of 16, and for each group and
// each 64-code K chunk c a 1 KiB block holding, for q = 0..3, the codes
// 64c + 16q .. +15 of the group's 16 tokens in token order -- byte
// ((((g*(k/64) + c)*4 + q)*16 + r)*16 + e) is code 64c + 16q + e of token
// 16g + r.  One v_mfma_i32_16x16x64_i8 operand is then one contiguous
// 1 KiB load (lane l takes bytes 16l..16l+15), where the row image spreads
// it over 16 half-used cache lines.  Tokens past t up to the next multiple
// of 16 are written as zero codes.
#include "kq_common.h"

namespace kq {

template <bool TILES>
__global__ __launch_bounds__(256) void quantize_q8k_kernel(const float *__restrict__ x, int64_t rows, int64_t t,
                                                           int nsb, int8_t *__restrict__ xq,
                                                           float *__restrict__ xs, int16_t *__restrict__ xbs)
{
    const int lane = threadIdx.x & 63;
    const int64_t chunk = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (chunk >= rows * nsb) return;  // whole wave exits together
    const int64_t row = chunk / nsb;
    const int sb = (int)(chunk - row * nsb);
    const bool real = row < t;  // uniform over the wave

    const float4 v = real ? reinterpret_cast<const float4 *>(x + chunk * QK)[lane] : make_float4(0, 0, 0, 0);
    int qsum;
    float d8;
    const uint32_t packed = q8k_chunk(v, qsum, d8);
    if constexpr (TILES) {
        const int64_t C = (int64_t)nsb * 4, g = row >> 4;
        const int r = (int)(row & 15), c = 4 * sb + (lane >> 4), q = (lane >> 2) & 3;
        const int64_t off = (((g * C + c) * 4 + q) * 16 + r) * 16 + 4 * (lane & 3);
        *reinterpret_cast<uint32_t *>(xq + off) = packed;
    } else {
        reinterpret_cast<uint32_t *>(xq + chunk * QK)[lane] = packed;
    }
    if (!real) return;
    // lanes 4g..4g+3 hold the 16 codes of group g
    if ((lane & 3) == 0) xbs[chunk * 16 + (lane >> 2)] = (int16_t)qsum;
    if (lane == 0) xs[chunk] = d8;
}

static int launch(bool tiles, const float *x, int64_t t, int64_t k, int8_t *xq, float *xs, int16_t *xbs,
                  hipStream_t stream)
{
    const int nsb = (int)(k / QK);
    const int64_t rows = tiles ? (t + 15) / 16 * 16 : t;
    const int per_block = 4;  // waves (chunks) per 256-thread workgroup
    const int64_t blocks = (rows * nsb + per_block - 1) / per_block;
    if (tiles)
        hipLaunchKernelGGL(quantize_q8k_kernel<true>, dim3((unsigned)blocks), dim3(64 * per_block), 0, stream, x,
                           rows, t, nsb, xq, xs, xbs);
    else
        hipLaunchKernelGGL(quantize_q8k_kernel<false>, dim3((unsigned)blocks), dim3(64 * per_block), 0, stream, x,
                           rows, t, nsb, xq, xs, xbs);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ELAUNCH;
}

int launch_quantize_q8k(const float *x, int64_t t, int64_t k, int8_t *xq, float *xs, int16_t *xbs,
                        hipStream_t stream)
{
    return launch(false, x, t, k, xq, xs, xbs, stream);
}

int launch_quantize_q8k_tiles(const float *x, int64_t t, int64_t k, int8_t *xq, float *xs, int16_t *xbs,
                              hipStream_t stream)
{
    return launch(true, x, t, k, xq, xs, xbs, stream);
}

}  // namespace kq
