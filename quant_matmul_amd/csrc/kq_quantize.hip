// kq_quantize.hip -- Q8_K activation quantiser (gfx950).
//
// Q8_K form (K-quant kernel arc page, "The pieces", kq v2 item; the k4 v2
// commit message): per 256 activations one float scale d8 = amax/127, int8
// codes a = round(x/d8), and an int16 sum of every 16 codes.  Both divisions
// are correctly rounded binary32 (__fdiv_rn) and the rounding is half to
// even (rintf), so the image is bit-identical to any IEEE implementation of
// the same definition.
//
// Small batches (a decode token): one wave per 256-value chunk, each lane
// owning 4 consecutive values (one 16-byte load, one 4-byte store), the
// chunk's amax a wave reduction and each 16-value bsum the sum over a quad
// of lanes -- the shortest critical path.  Large batches use the wide form
// below (four chunks per wave, 16 values per lane).
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

// a / b for 0 <= a and 0 < b < 2^31; a 32-bit division whenever a < 2^32
// (every realistic grid: the 64-bit one is a long instruction sequence ahead
// of the first load)
__device__ inline int64_t udiv(int64_t a, int b)
{
    if (a <= (int64_t)UINT32_MAX) return (int64_t)((uint32_t)a / (uint32_t)b);
    return a / b;
}

template <bool TILES, bool GATHER>
__global__ __launch_bounds__(256) void quantize_q8k_kernel(const float *__restrict__ x, int64_t t,
                                                           const int32_t *__restrict__ src, int64_t m,
                                                           int64_t rows, int nsb, int8_t *__restrict__ xq,
                                                           float *__restrict__ xs, int16_t *__restrict__ xbs)
{
    const int lane = threadIdx.x & 63;
    const int64_t chunk = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (chunk >= rows * nsb) return;  // whole wave exits together
    const int64_t row = udiv(chunk, nsb);
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

// Wide form, for large batches: lane l of a wave holds values 16j .. 16j+15
// (j = l % 16) of chunk l / 16 of the wave, so its 16 codes are one bsum
// group and one 16-byte piece of either image (the tile form's four chunks
// are four consecutive tokens of one superblock, whose pieces are
// adjacent), and the chunk's amax is a reduction over a 16-lane DPP row.
// Measured against the one-chunk-per-wave form: 10.8 -> 7.4 us for the
// 512 x 9728 tile image, but 0.3 us slower for one token, whose 16 serial
// divisions per lane lengthen the critical path.
template <bool TILES, bool GATHER>
__global__ __launch_bounds__(256) void quantize_q8k_wide_kernel(const float *__restrict__ x, int64_t t,
                                                           const int32_t *__restrict__ src, int64_t m,
                                                           int64_t rows, int nsb, int8_t *__restrict__ xq,
                                                           float *__restrict__ xs, int16_t *__restrict__ xbs)
{
    const int lane = threadIdx.x & 63, sub = lane >> 4, j = lane & 15;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    int64_t row;
    int sb;
    if constexpr (TILES) {
        // four consecutive tokens of one superblock: their code pieces are
        // adjacent in the tile image
        const int64_t quad = udiv(wave, nsb);
        sb = (int)(wave - quad * nsb);
        row = quad * 4 + sub;
        if (quad * 4 >= rows) return;  // whole wave exits together
    } else {
        const int64_t chunk = wave * 4 + sub;
        row = udiv(chunk, nsb);
        sb = (int)(chunk - row * nsb);
        if (wave * 4 >= rows * nsb) return;
    }
    const bool inrange = row < rows;
    const bool real = inrange && row < m;
    int64_t srow = row;
    if constexpr (GATHER) srow = real ? (int64_t)src[row] : -1;
    const bool data = real && srow >= 0 && srow < t;
    float v[16];
    {
        const float4 *p = reinterpret_cast<const float4 *>(x + (srow * nsb + sb) * QK + 16 * j);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 f = data ? p[i] : make_float4(0, 0, 0, 0);
            v[4 * i] = f.x;
            v[4 * i + 1] = f.y;
            v[4 * i + 2] = f.z;
            v[4 * i + 3] = f.w;
        }
    }
    int qsum;
    float d8;
    const uint4 piece = q8k_piece16(v, qsum, d8);
    if (!inrange) return;
    if constexpr (TILES) {
        // codes 16j..16j+15 of superblock sb: K chunk c = 8*sb + j/2, half q = j & 1
        const int64_t g = row >> 5;
        const int r = (int)(row & 31), q = j & 1;
        const int64_t c = (int64_t)sb * 8 + (j >> 1);
        *reinterpret_cast<uint4 *>(xq + ((g * nsb * 8 + c) * 64 + q * 32 + r) * 16) = piece;
        _Float16 *bt = reinterpret_cast<_Float16 *>(xbs);
        bt[((g * nsb + sb) * 64 + (j >> 3) * 32 + r) * 8 + (j & 7)] = (_Float16)qsum;
        if (real && j == 0) xs[row * nsb + sb] = d8;
    } else {
        const int64_t chunk = row * nsb + sb;
        *reinterpret_cast<uint4 *>(xq + chunk * QK + 16 * j) = piece;
        xbs[chunk * 16 + j] = (int16_t)qsum;
        if (j == 0) xs[chunk] = d8;
    }
}

template <bool TILES, bool GATHER>
static int launch(const float *x, int64_t t, const int32_t *src, int64_t m, int64_t k, int8_t *xq, float *xs,
                  int16_t *xbs, hipStream_t stream)
{
    const int nsb = (int)(k / QK);
    const int64_t rows = TILES ? (m + 31) / 32 * 32 : m;
    const int per_block = 4;  // waves per 256-thread workgroup
    const int64_t chunks = rows * nsb;
    if (chunks >= 2048) {
        // wide form: four chunks per wave
        const int64_t waves = TILES ? rows / 4 * nsb : (chunks + 3) / 4;
        const int64_t blocks = (waves + per_block - 1) / per_block;
        hipLaunchKernelGGL((quantize_q8k_wide_kernel<TILES, GATHER>), dim3((unsigned)blocks), dim3(64 * per_block), 0,
                           stream, x, t, src, m, rows, nsb, xq, xs, xbs);
    } else {
        const int64_t blocks = (chunks + per_block - 1) / per_block;
        hipLaunchKernelGGL((quantize_q8k_kernel<TILES, GATHER>), dim3((unsigned)blocks), dim3(64 * per_block), 0,
                           stream, x, t, src, m, rows, nsb, xq, xs, xbs);
    }
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

namespace kq {

// Row image -> tile image (the GEMM's operand order), for callers holding the
// image kq_quantize_q8k writes.  Thread i writes the i-th 16-byte piece of the
// tile codes, so the stores are one linear stream: piece i is codes
// 32c + 16q .. +15 of token 32g + r, with i = ((g*(k/32) + c)*2 + q)*32 + r.
// Those 16 codes are exactly bsum group 2c + q of the token, whose int16 sum
// goes to its f16 slot (exact: |bsum| <= 2032).  Tokens m .. rows-1 (the
// padding up to a multiple of 32) get zero codes and zero bsums.  Only bytes
// move, so the result is bit-identical to kq_quantize_q8k_tiles on the same
// activations.
__global__ __launch_bounds__(256) void relay_tiles_kernel(const int8_t *__restrict__ xq,
                                                          const int16_t *__restrict__ xbs, int64_t m, int64_t rows,
                                                          int nsb, int8_t *__restrict__ xqt,
                                                          _Float16 *__restrict__ xbt)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t kc = (int64_t)nsb * 8;  // 32-code chunks per row
    if (i >= rows * kc * 2) return;
    const int r = (int)(i & 31);
    const int64_t rest = i >> 5;
    const int q = (int)(rest & 1);
    const int64_t gc = rest >> 1;
    const int64_t g = gc / kc, c = gc - g * kc;
    const int64_t row = g * 32 + r;
    const int64_t p = 2 * c + q;  // 16-code piece of the row = its bsum group
    uint4 v = make_uint4(0, 0, 0, 0);
    int b = 0;
    if (row < m) {
        v = *reinterpret_cast<const uint4 *>(xq + row * kc * 32 + 16 * p);
        b = xbs[row * kc * 2 + p];
    }
    *reinterpret_cast<uint4 *>(xqt + i * 16) = v;
    const int64_t s = p >> 4;
    const int j = (int)(p & 15);
    xbt[((g * nsb + s) * 64 + (j >> 3) * 32 + r) * 8 + (j & 7)] = (_Float16)b;
}

int launch_relay_tiles(const int8_t *xq, const int16_t *xbs, int64_t m, int64_t k, int8_t *xqt, uint16_t *xbt,
                       hipStream_t stream)
{
    const int nsb = (int)(k / QK);
    const int64_t rows = (m + 31) / 32 * 32;
    const int64_t threads = rows * (k / 16);
    hipLaunchKernelGGL(relay_tiles_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, xq, xbs, m,
                       rows, nsb, xqt, reinterpret_cast<_Float16 *>(xbt));
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ELAUNCH;
}

}  // namespace kq
