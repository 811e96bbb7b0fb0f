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
// Two layouts.  The row image is xq[t][k], xbs[t][k/16] int16.  The tile
// image feeds the GEMM's MFMA operands directly: tokens in groups of 32;
//  * codes: for group g and 32-code K chunk c a contiguous 1 KiB block in
//    which byte ((q*32 + r)*16 + e), q in 0..1, is code 32c + 16q + e of
//    token 32g + r -- the A operand of v_mfma_i32_32x32x32_i8, lane l = 32q
//    + r taking bytes 16l..16l+15;
//  * bsums: for group g and superblock s a 1 KiB block of f16 in which
//    element (q*32 + r)*8 + e is bsum 8q + e of token 32g + r (exact: |bsum|
//    <= 2032) -- the A operand of v_mfma_f32_32x32x16_f16.
// One operand is then one coalesced 1 KiB load with no conversion, where
// row-major codes spread it over 32 partly used cache lines.  Tokens past t
// up to the next multiple of 32 get zero codes and zero bsums.
//
// The gather form fills the tile image of a mixture-of-experts layer: image
// row i is the Q8_K of activation row src[i] (the tokens routed to each
// expert, each expert's rows padded to whole tiles), and an index outside
// the activation rows gives a zero row.
#include "kq_common.h"

namespace kq {

template <bool TILES, bool GATHER>
__global__ __launch_bounds__(256) void quantize_q8k_kernel(const float *__restrict__ x, int64_t t,
                                                           const int32_t *__restrict__ src, int64_t m,
                                                           int64_t rows, int nsb, int8_t *__restrict__ xq,
                                                           float *__restrict__ xs, int16_t *__restrict__ xbs)
{
    const int lane = threadIdx.x & 63;
    const int64_t chunk = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (chunk >= rows * nsb) return;  // whole wave exits together
    const int64_t row = chunk / nsb;
    const int sb = (int)(chunk - row * nsb);
    // image row `row` (< m: a real row, else tile padding) quantises source
    // row srow of x; a gather index outside [0, t) gives a zero row
    const bool real = row < m;  // uniform over the wave
    int64_t srow = row;
    if constexpr (GATHER) srow = real ? (int64_t)src[row] : -1;
    const bool data = real && srow >= 0 && srow < t;

    const float4 v = data ? reinterpret_cast<const float4 *>(x + (srow * nsb + sb) * QK)[lane]
                          : make_float4(0, 0, 0, 0);
    int qsum;
    float d8;
    const uint32_t packed = q8k_chunk(v, qsum, d8);
    if constexpr (TILES) {
        // lane owns codes 4*lane..+3 of the superblock: chunk c = 8*sb +
        // lane/8, half q = (lane/4) & 1, byte 4*(lane & 3) of the piece
        const int64_t g = row >> 5;
        const int r = (int)(row & 31), q = (lane >> 2) & 1;
        const int64_t c = (int64_t)sb * 8 + (lane >> 3);
        const int64_t off = ((g * nsb * 8 + c) * 64 + q * 32 + r) * 16 + 4 * (lane & 3);
        *reinterpret_cast<uint32_t *>(xq + off) = packed;
        // bsum j = lane/4 of this superblock, as f16, in the f16 operand order
        if ((lane & 3) == 0) {
            const int j = lane >> 2;
            _Float16 *bt = reinterpret_cast<_Float16 *>(xbs);
            bt[((g * nsb + sb) * 64 + (j >> 3) * 32 + r) * 8 + (j & 7)] = (_Float16)qsum;
        }
        if (real && lane == 0) xs[chunk] = d8;
    } else {
        reinterpret_cast<uint32_t *>(xq + chunk * QK)[lane] = packed;
        // lanes 4g..4g+3 hold the 16 codes of group g
        if ((lane & 3) == 0) xbs[chunk * 16 + (lane >> 2)] = (int16_t)qsum;
        if (lane == 0) xs[chunk] = d8;
    }
}

template <bool TILES, bool GATHER>
static int launch(const float *x, int64_t t, const int32_t *src, int64_t m, int64_t k, int8_t *xq, float *xs,
                  int16_t *xbs, hipStream_t stream)
{
    const int nsb = (int)(k / QK);
    const int64_t rows = TILES ? (m + 31) / 32 * 32 : m;
    const int per_block = 4;  // waves (chunks) per 256-thread workgroup
    const int64_t blocks = (rows * nsb + per_block - 1) / per_block;
    hipLaunchKernelGGL((quantize_q8k_kernel<TILES, GATHER>), dim3((unsigned)blocks), dim3(64 * per_block), 0, stream,
                       x, t, src, m, rows, nsb, xq, xs, xbs);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ELAUNCH;
}

int launch_quantize_q8k(const float *x, int64_t t, int64_t k, int8_t *xq, float *xs, int16_t *xbs,
                        hipStream_t stream)
{
    return launch<false, false>(x, t, nullptr, t, k, xq, xs, xbs, stream);
}

int launch_quantize_q8k_tiles(const float *x, int64_t t, int64_t k, int8_t *xq, float *xs, int16_t *xbs,
                              hipStream_t stream)
{
    return launch<true, false>(x, t, nullptr, t, k, xq, xs, xbs, stream);
}

int launch_quantize_q8k_tiles_gather(const float *x, int64_t t, const int32_t *src, int64_t m, int64_t k,
                                     int8_t *xq, float *xs, int16_t *xbs, hipStream_t stream)
{
    return launch<true, true>(x, t, src, m, k, xq, xs, xbs, stream);
}

}  // namespace kq
