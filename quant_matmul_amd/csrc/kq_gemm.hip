// kq_gemm.hip -- prefill GEMM (m tokens x n rows) on gfx950 int8 MFMA.
//
// Same contract as the GEMV: per (token, row, superblock) the exact int32
// partials P (and M), then one float fold (K-quant kernel arc page, "The
// pieces", kq v2 item).  The MI355X design:
//
//  * Panel unpack, once per (row panel, token block).  As in the page's kq
//    v3 panel scratch ("The pieces", kq v3 item: unpack the packed planes
//    once per (group, token-block) and amortise it over the token block),
//    each workgroup unpacks the superblock of its 32 weight rows into LDS
//    once and reuses it for all 256 tokens.  What lands in LDS is not the
//    raw quant but the sub-scale-folded weight w' = sc*q (Q4_K/Q5_K,
//    0..1953) or sc*(q-32) (Q6_K, -4064..4096), split into two int8 digits
//    w' = 128*h + l with l in 0..127: the MFMA cannot apply a per-row,
//    per-sub-block scale, so folding it into the operand is what keeps the
//    per-sub-block integer fold on the matrix cores.
//  * Dense contraction: v_mfma_i32_16x16x64_i8, a high-digit pass, a shift
//    by 7, a low-digit pass into the same int32 accumulator -- which then
//    holds P = sum_j sc_j * dot_j exactly (|P| < 2^27).
//  * Min term: M = sum_g m_{g/2} * bsum_g is a 16-deep contraction per
//    superblock, done on v_mfma_f32_16x16x16_f16 (bsums |.| <= 2032 and
//    m <= 63 are exact in f16, and |M| < 2^24 keeps the f32 sum exact).
//  * Epilogue per superblock: acc += d8 * (d*P - dmin*M).
//
// A operand.  The codes come from the tile image of the Q8_K quantiser
// (16 tokens x 64 codes per contiguous KiB), so each A fragment is one fully
// coalesced 1 KiB load; with row-major codes the same fragment touches 16
// half-used cache lines, and the L2-to-L1 traffic that costs, not the
// matrix cores, bounded the kernel.  Codes and bsums are read through
// buffer resources based at the workgroup's first token: tokens past the
// image read as zero and their outputs are never stored.
//
// Pipeline.  A workgroup is 4 waves over a 256-token x 32-row tile; each
// wave owns 64 tokens x 32 rows (4 x 2 MFMA tiles of 16x16).  Per
// superblock s the wave's codes sit in registers, the digit panel in one of
// two LDS buffers; while the high-digit MFMAs of s run, the wave unpacks its
// share of superblock s+1 (whose packed bytes were prefetched) into the
// other buffer, so the VALU unpack overlaps the matrix pipe, and each
// 64-deep K step of the codes is refilled with superblock s+1 as soon as
// its low-digit MFMAs are issued.  One barrier per superblock.
#include "kq_common.h"

namespace kq {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int LDS_STRIDE = 272;  // bytes per digit row: 256 + 16 pad

namespace {

// Split four folded weights (16-bit lanes e = w'0 | w'2 << 16 and
// o = w'1 | w'3 << 16, each lane value in [0, 65535]) into their low digits
// (bits 0..6) and high digits (bits 7..13), packed as four bytes each.
__device__ inline void split_digits(uint32_t e, uint32_t o, uint32_t &hi, uint32_t &lo)
{
    lo = (e & 0x007F007Fu) | ((o & 0x007F007Fu) << 8);
    hi = ((e >> 7) & 0x007F007Fu) | (((o >> 7) & 0x007F007Fu) << 8);
}

// Four unsigned quants (one per byte of q, each <= 31) times scale sc
// (0..63): the digits of sc*q.
__device__ inline void digits_q45(uint32_t q, int sc, uint32_t &hi, uint32_t &lo)
{
    // each 16-bit lane <= 31*63, and both factors fit 24 bits
    const uint32_t e = (uint32_t)__umul24(q & 0x00FF00FFu, (uint32_t)sc);
    const uint32_t o = (uint32_t)__umul24((q >> 8) & 0x00FF00FFu, (uint32_t)sc);
    split_digits(e, o, hi, lo);
}

// Four Q6_K quants (bytes 0..63) with signed scale sc: the digits of
// w' = sc*(q-32).  Each 16-bit lane is formed as w' + 4096 in [32, 8192]
// (q*sc + 4096 - 32*sc); the integer sum of the two lanes is exact, so the
// lanes never borrow.  The low digit of w' + 4096 is that of w' (4096 is a
// multiple of 128), the high digit is 32 too large: it is taken back per
// byte with a borrow-free byte subtraction, leaving a signed byte.
__device__ inline void digits_q6(uint32_t q, int sc, uint32_t &hi, uint32_t &lo)
{
    const int bias = (4096 - 32 * sc) * 0x00010001;
    const uint32_t e = (uint32_t)(__mul24((int)(q & 0x00FF00FFu), sc) + bias);
    const uint32_t o = (uint32_t)(__mul24((int)((q >> 8) & 0x00FF00FFu), sc) + bias);
    uint32_t hu;
    split_digits(e, o, hu, lo);
    hi = ((hu | 0x80808080u) - 0x20202020u) ^ 0x80808080u;
}

// Half share: 32 weights of a superblock row, one unpack task.  Task
// h = 2c + half of a Q4_K/Q5_K row covers quant bytes 32c + 16*half .. +15:
// their low nibbles are weights 64c + 16*half + 0..15 (sub-block 2c), their
// high nibbles weights 64c + 32 + 16*half + 0..15 (sub-block 2c+1).  Task
// h = 2c + half of a Q6_K row (c = 2hh + u) covers low-array bytes
// 64hh + 32u + 16*half .. +15: weights 128hh + 32u + 16*half + 0..15
// (sub-block 8hh + 2u + half) and the same + 64 (sub-block 8hh + 2u + 4 + half).
template <int FMT>
struct Half;
template <>
struct Half<KQ_Q4_K> {
    uint4 h, q;
};
template <>
struct Half<KQ_Q5_K> {
    uint4 h, q, qh;
};
template <>
struct Half<KQ_Q6_K> {
    uint4 l, hq;
    uint2 s8;
    uint32_t d;
};

__device__ inline void load_half(Half<KQ_Q4_K> &r, const uint8_t *__restrict__ w, const Planes &pl, int64_t sb, int h)
{
    r.h = *reinterpret_cast<const uint4 *>(w + pl.off[0] + sb * 16);
    r.q = *reinterpret_cast<const uint4 *>(w + pl.off[1] + sb * 128 + 16 * h);
}
__device__ inline void load_half(Half<KQ_Q5_K> &r, const uint8_t *__restrict__ w, const Planes &pl, int64_t sb, int h)
{
    r.h = *reinterpret_cast<const uint4 *>(w + pl.off[0] + sb * 16);
    r.qh = *reinterpret_cast<const uint4 *>(w + pl.off[1] + sb * 32 + 16 * (h & 1));
    r.q = *reinterpret_cast<const uint4 *>(w + pl.off[2] + sb * 128 + 16 * h);
}
__device__ inline void load_half(Half<KQ_Q6_K> &r, const uint8_t *__restrict__ w, const Planes &pl, int64_t sb, int h)
{
    const int c = h >> 1, half = h & 1, hh = c >> 1;
    r.l = *reinterpret_cast<const uint4 *>(w + pl.off[0] + sb * 128 + 16 * h);
    r.hq = *reinterpret_cast<const uint4 *>(w + pl.off[1] + sb * 64 + 32 * hh + 16 * half);
    r.s8 = *reinterpret_cast<const uint2 *>(w + pl.off[2] + sb * 16 + 8 * hh);
    r.d = *reinterpret_cast<const uint16_t *>(w + pl.off[3] + sb * 2);
}

__device__ inline void store_half(int8_t *wh, int8_t *wl, int r, int k0, const uint32_t (&h)[4], const uint32_t (&l)[4])
{
    *reinterpret_cast<uint4 *>(wh + r * LDS_STRIDE + k0) = make_uint4(h[0], h[1], h[2], h[3]);
    *reinterpret_cast<uint4 *>(wl + r * LDS_STRIDE + k0) = make_uint4(l[0], l[1], l[2], l[3]);
}

__device__ inline void unpack_half(const Half<KQ_Q6_K> &rw, bool valid, int r, int h, int8_t *wh, int8_t *wl,
                                   _Float16 *, float *dn, float *dmn)
{
    const int c = h >> 1, half = h & 1, hh = c >> 1, u = c & 1;
    const uint32_t lw[4] = {rw.l.x, rw.l.y, rw.l.z, rw.l.w};
    const uint32_t hw[4] = {rw.hq.x, rw.hq.y, rw.hq.z, rw.hq.w};
    const uint2 s8 = valid ? rw.s8 : make_uint2(0, 0);
    const int slo = (int8_t)byte_of(s8.x, 2 * u + half), shi = (int8_t)byte_of(s8.y, 2 * u + half);
    uint32_t h0[4], l0[4], h1[4], l1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (lw[i] & 0x0F0F0F0Fu) | (((hw[i] >> (2 * u)) & 0x03030303u) << 4);
        const uint32_t hi = ((lw[i] >> 4) & 0x0F0F0F0Fu) | (((hw[i] >> (2 * u + 4)) & 0x03030303u) << 4);
        digits_q6(lo, slo, h0[i], l0[i]);
        digits_q6(hi, shi, h1[i], l1[i]);
    }
    const int k0 = 128 * hh + 32 * u + 16 * half;
    store_half(wh, wl, r, k0, h0, l0);
    store_half(wh, wl, r, k0 + 64, h1, l1);
    if (h == 0) {
        dn[r] = valid ? f16_bits_to_float(rw.d) : 0.0f;
        dmn[r] = 0.0f;
    }
}

template <int FMT>
__device__ inline void unpack_half(const Half<FMT> &rw, bool valid, int r, int h, int8_t *wh, int8_t *wl,
                                   _Float16 *mexp, float *dn, float *dmn)
{
    const int c = h >> 1, half = h & 1;
    const uint4 hd = valid ? rw.h : make_uint4(0, 0, 0, 0);
    const uint32_t qw[4] = {rw.q.x, rw.q.y, rw.q.z, rw.q.w};
    int sc0, m0, sc1, m1;
    scale_min_6bit(hd.y, hd.z, hd.w, 2 * c, sc0, m0);
    scale_min_6bit(hd.y, hd.z, hd.w, 2 * c + 1, sc1, m1);
    uint32_t h0[4], l0[4], h1[4], l1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t lo = qw[i] & 0x0F0F0F0Fu, hi = (qw[i] >> 4) & 0x0F0F0F0Fu;
        if constexpr (FMT == KQ_Q5_K) {
            const uint32_t hb = i == 0 ? rw.qh.x : i == 1 ? rw.qh.y : i == 2 ? rw.qh.z : rw.qh.w;
            lo |= ((hb >> (2 * c)) & 0x01010101u) << 4;
            hi |= ((hb >> (2 * c + 1)) & 0x01010101u) << 4;
        }
        digits_q45(lo, sc0, h0[i], l0[i]);
        digits_q45(hi, sc1, h1[i], l1[i]);
    }
    const int k0 = 64 * c + 16 * half;
    store_half(wh, wl, r, k0, h0, l0);
    store_half(wh, wl, r, k0 + 32, h1, l1);
    if (half == 0) {
        // min of sub-block j pairs with bsums 2j and 2j+1
        _Float16 *me = mexp + r * 16 + 4 * c;
        me[0] = me[1] = (_Float16)m0;
        me[2] = me[3] = (_Float16)m1;
    }
    if (h == 0) {
        dn[r] = f16_bits_to_float(hd.x & 0xFFFFu);
        dmn[r] = f16_bits_to_float(hd.x >> 16);
    }
}

// Workgroup tile index -> (row panel, token block), grouping the token
// blocks of one row panel on one XCD (workgroup b runs on XCD b % 8), so the
// panel's packed planes are fetched into that XCD's L2 once.
__device__ inline void tile_of(int b, int G, int mtiles, int &nt, int &mt)
{
    const int per = G / 8;
    int L = b;
    if (b < per * 8) L = (b % 8) * per + b / 8;
    nt = L / mtiles;
    mt = L % mtiles;
}

}  // namespace

template <int FMT, bool PART>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const uint8_t *__restrict__ w, int64_t n, int nsb,
                                                      const int8_t *__restrict__ xq, const float *__restrict__ xs,
                                                      const int16_t *__restrict__ xbs, int64_t mtok,
                                                      float *__restrict__ y, int32_t *__restrict__ Pout,
                                                      int32_t *__restrict__ Mout, int mtiles)
{
    constexpr int BM = 256, BN = 32;
    static_assert(BN * 8 == 256, "one 32-weight unpack task per thread");
    __shared__ __align__(16) int8_t wh[2][BN * LDS_STRIDE];
    __shared__ __align__(16) int8_t wl[2][BN * LDS_STRIDE];
    __shared__ __align__(16) _Float16 mexp[2][BN * 16];
    __shared__ float dn[2][BN], dmn[2][BN];
    __shared__ __align__(16) float d8s[2][BM];

    int nt, mt;
    tile_of(blockIdx.x, gridDim.x, mtiles, nt, mt);
    const int64_t n0 = (int64_t)nt * BN, m0 = (int64_t)mt * BM;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wm = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    const int64_t K = (int64_t)nsb * QK, KB = K / 16;
    const Planes pl = planes_of(FMT, n, nsb);

    // unpack task of this thread (rows past n read row n-1, unpack as 0)
    const int64_t wr = n0 + (tid >> 3);
    const bool wvalid = wr < n;
    const int64_t wrow = (wvalid ? wr : n - 1) * nsb;
    Half<FMT> raw;
    const int64_t t_d8 = m0 + tid;
    const float *xs_row = xs + (t_d8 < mtok ? t_d8 : mtok - 1) * nsb;
    float d8n = 0.0f;
    auto load_w = [&](int s) {
        load_half(raw, w, pl, wrow + s, tid & 7);
        d8n = t_d8 < mtok ? xs_row[s] : 0.0f;
    };
    auto unpack_w = [&](int b) {
        unpack_half(raw, wvalid, tid >> 3, tid & 7, wh[b], wl[b], mexp[b], dn[b], dmn[b]);
        d8s[b][tid] = d8n;
    };

    // Codes (A operand, tile image: 16 tokens x 64 codes per KiB) and bsums
    // (f16 A operand of the min term, row-major) of the wave's 64 tokens.
    // The tile image holds tokens up to m rounded up to 16.
    const uint64_t a_bytes = (uint64_t)(((mtok + 15) & ~(int64_t)15) - m0) * (uint64_t)K;
    const uint64_t b_bytes = (uint64_t)(mtok - m0) * (uint64_t)KB * 2;
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xq + m0 * K), 0, (int)(uint32_t)(a_bytes < 0xFFFFFFFFu ? a_bytes : 0xFFFFFFFFu), 0x00020000);
    const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xbs + m0 * KB), 0, (int)(uint32_t)(b_bytes < 0xFFFFFFFFu ? b_bytes : 0xFFFFFFFFu), 0x00020000);
    // 32-bit offsets: the caller bounds k so that 256 tokens of codes < 2^31
    int aoff[4], boff[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        aoff[mi] = (wm * 4 + mi) * 16 * (int)K + 16 * lane;
        boff[mi] = (wm * 64 + mi * 16 + l16) * (int)KB * 2 + 8 * lq;
    }
    i32x4 A[4][4];
    f16x4 Ab[4];
    auto load_a = [&](int s, int ks) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            A[mi][ks] = __builtin_bit_cast(
                i32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, aoff[mi] + (s * 4 + ks) * 1024, 0, 0));
    };
    auto load_bs = [&](int s) {
        if constexpr (FMT != KQ_Q6_K) {
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const i32x2 bq =
                    __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(rB, boff[mi] + s * 32, 0, 0));
                Ab[mi][0] = (_Float16)(int16_t)(bq.x & 0xFFFF);
                Ab[mi][1] = (_Float16)(int16_t)(bq.x >> 16);
                Ab[mi][2] = (_Float16)(int16_t)(bq.y & 0xFFFF);
                Ab[mi][3] = (_Float16)(int16_t)(bq.y >> 16);
            }
        }
    };

    f32x4 accf[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) accf[mi][0] = accf[mi][1] = f32x4{};

    load_w(0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) load_a(0, ks);
    load_bs(0);
    unpack_w(0);
    if (nsb > 1) load_w(1);
    __syncthreads();

    for (int s = 0; s < nsb; ++s) {
        const int b = s & 1;
        i32x4 acc[4][2];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) acc[mi][0] = acc[mi][1] = i32x4{};
        // high-digit pass
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int nj = 0; nj < 2; ++nj) {
                const i32x4 B = *reinterpret_cast<const i32x4 *>(wh[b] + (nj * 16 + l16) * LDS_STRIDE + 64 * ks + 16 * lq);
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
                    acc[mi][nj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[mi][ks], B, acc[mi][nj], 0, 0, 0);
            }
        }
        // the unpack of the next superblock overlaps these MFMAs
        if (s + 1 < nsb) unpack_w(b ^ 1);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            acc[mi][0] = acc[mi][0] * 128;
            acc[mi][1] = acc[mi][1] * 128;
        }
        // low-digit pass; each 64-deep K step of the codes is dead after it
        // and is refilled with superblock s+1 at once
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int nj = 0; nj < 2; ++nj) {
                const i32x4 B = *reinterpret_cast<const i32x4 *>(wl[b] + (nj * 16 + l16) * LDS_STRIDE + 64 * ks + 16 * lq);
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
                    acc[mi][nj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[mi][ks], B, acc[mi][nj], 0, 0, 0);
            }
            if (s + 1 < nsb) load_a(s + 1, ks);
        }
        // the one float fold of superblock s; the min term (exact f16 MFMA
        // over the 16 bsums) is formed per 16-row column just before it
#pragma unroll
        for (int nj = 0; nj < 2; ++nj) {
            const int rl = nj * 16 + l16;
            const float dv = dn[b][rl], dm = dmn[b][rl];
            const int64_t col = n0 + rl;
            f32x4 mf[4];
            if constexpr (FMT != KQ_Q6_K) {
                const f16x4 Bm = *reinterpret_cast<const f16x4 *>(mexp[b] + rl * 16 + 4 * lq);
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
                    mf[mi] = __builtin_amdgcn_mfma_f32_16x16x16f16(Ab[mi], Bm, f32x4{}, 0, 0, 0);
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tl = wm * 64 + mi * 16 + 4 * lq + i;
                    const float Pf = (float)acc[mi][nj][i];
                    float u;
                    if constexpr (FMT == KQ_Q6_K) u = dv * Pf;
                    else u = fmaf(dv, Pf, -(dm * mf[mi][i]));
                    accf[mi][nj][i] = fmaf(d8s[b][tl], u, accf[mi][nj][i]);
                    if (PART) {
                        const int64_t t = m0 + tl;
                        if (t < mtok && col < n) {
                            const int64_t o = (t * n + col) * nsb + s;
                            Pout[o] = acc[mi][nj][i];
                            if (Mout) {
                                if constexpr (FMT == KQ_Q6_K) Mout[o] = 0;
                                else Mout[o] = (int)mf[mi][i];
                            }
                        }
                    }
                }
            }
        }
        if (s + 1 < nsb) load_bs(s + 1);
        if (s + 2 < nsb) load_w(s + 2);
        __syncthreads();  // panel s+1 complete; panel s free for s+2
    }

#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t t = m0 + wm * 64 + mi * 16 + 4 * lq + i;
            if (t >= mtok) continue;
#pragma unroll
            for (int nj = 0; nj < 2; ++nj) {
                const int64_t col = n0 + nj * 16 + l16;
                if (col < n) y[t * n + col] = accf[mi][nj][i];
            }
        }
}

template <int FMT>
static void launch_fmt(bool part, int64_t n, int nsb, const uint8_t *w, const int8_t *xq, const float *xs,
                       const int16_t *xbs, int64_t m, float *y, int32_t *P, int32_t *M, hipStream_t st)
{
    constexpr int BM = 256, BN = 32;
    const int64_t ntiles = (n + BN - 1) / BN, mtiles = (m + BM - 1) / BM;
    const dim3 g((unsigned)(ntiles * mtiles)), b(256);
    if (part)
        hipLaunchKernelGGL((gemm_kernel<FMT, true>), g, b, 0, st, w, n, nsb, xq, xs, xbs, m, y, P, M, (int)mtiles);
    else
        hipLaunchKernelGGL((gemm_kernel<FMT, false>), g, b, 0, st, w, n, nsb, xq, xs, xbs, m, y, P, M, (int)mtiles);
}

int launch_gemm(int fmt, const void *w, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                const int16_t *xbs, int64_t m, float *y, int32_t *P, int32_t *M, hipStream_t st)
{
    const int nsb = (int)(k / QK);
    const uint8_t *wb = (const uint8_t *)w;
    const bool part = P != nullptr;
    if (fmt == KQ_Q4_K) launch_fmt<KQ_Q4_K>(part, n, nsb, wb, xq, xs, xbs, m, y, P, M, st);
    else if (fmt == KQ_Q5_K) launch_fmt<KQ_Q5_K>(part, n, nsb, wb, xq, xs, xbs, m, y, P, M, st);
    else launch_fmt<KQ_Q6_K>(part, n, nsb, wb, xq, xs, xbs, m, y, P, M, st);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ELAUNCH;
}

}  // namespace kq
