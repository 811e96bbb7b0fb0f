// kq_gemm.hip -- prefill GEMM (m tokens x n rows) on gfx950 int8 MFMA.
//
// Same contract as the GEMV: per (token, row, superblock) the exact int32
// partials P (and M), then one float fold (K-quant kernel arc page, "The
// pieces", kq v2 item).  The MI355X design:
//
//  * Panel unpack, once per (row panel, token block).  As in the page's kq
//    v3 panel scratch ("The pieces", kq v3 item: unpack the packed planes
//    once per (group, token-block) and amortise it over the token block),
//    each workgroup unpacks the superblock of its BN weight rows into LDS
//    once and reuses it for all BM tokens.  What lands in LDS is not the raw
//    quant but the sub-scale-folded weight w' = sc*q (Q4_K/Q5_K, 0..1953) or
//    sc*(q-32) (Q6_K, -4064..4096), split into two int8 digits
//    w' = 128*h + l with l in 0..127: the MFMA cannot apply a per-row,
//    per-sub-block scale, so folding it into the operand is what keeps the
//    per-sub-block integer fold on the matrix cores.
//  * Dense contraction: v_mfma_i32_32x32x32_i8, a high-digit pass, a shift by
//    7, a low-digit pass into the same int32 accumulator -- which then holds
//    P = sum_j sc_j * dot_j exactly (|P| < 2^27).
//  * Min term: M = sum_g m_{g/2} * bsum_g is a 16-deep contraction per
//    superblock, done on one v_mfma_f32_32x32x16_f16 (bsums |.| <= 2032 and
//    m <= 63 are exact in f16, and |M| < 2^24 keeps the f32 sum exact).
//  * Epilogue per superblock: acc += d8 * (d*P - dmin*M).
//
// Wave tile 64 tokens x 32*TN rows (2 x TN MFMA tiles); WM x WN waves.
#include "kq_common.h"

namespace kq {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

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
    const uint32_t e = (q & 0x00FF00FFu) * (uint32_t)sc;
    const uint32_t o = ((q >> 8) & 0x00FF00FFu) * (uint32_t)sc;
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
    const uint32_t e = (uint32_t)((int)(q & 0x00FF00FFu) * sc + bias);
    const uint32_t o = (uint32_t)((int)((q >> 8) & 0x00FF00FFu) * sc + bias);
    uint32_t hu;
    split_digits(e, o, hu, lo);
    hi = ((hu | 0x80808080u) - 0x20202020u) ^ 0x80808080u;
}

template <int FMT>
__device__ inline void store_digits(int8_t *wh, int8_t *wl, int r, int k0, const uint32_t (&h)[8],
                                    const uint32_t (&l)[8])
{
    uint4 *ph = reinterpret_cast<uint4 *>(wh + r * LDS_STRIDE + k0);
    uint4 *pl = reinterpret_cast<uint4 *>(wl + r * LDS_STRIDE + k0);
    ph[0] = make_uint4(h[0], h[1], h[2], h[3]);
    ph[1] = make_uint4(h[4], h[5], h[6], h[7]);
    pl[0] = make_uint4(l[0], l[1], l[2], l[3]);
    pl[1] = make_uint4(l[4], l[5], l[6], l[7]);
}

// Unpack 64 weights of row r (task c of 4) of superblock sb into the digit
// panel.  Q4_K/Q5_K task c covers sub-blocks 2c and 2c+1 (k = 64c..64c+63);
// Q6_K task c = 2h + u covers k = 128h + 32u + 0..31 and + 64 + 0..31.
template <int FMT>
__device__ inline void unpack_task(const uint8_t *__restrict__ w, const Planes &pl, int64_t sb, bool valid,
                                   int r, int c, int8_t *wh, int8_t *wl, _Float16 *mexp, float *dn, float *dmn)
{
    uint32_t h0[8], l0[8], h1[8], l1[8];
    if (FMT == KQ_Q6_K) {
        const int hh = c >> 1, u = c & 1;
        uint32_t lo[8], hi[8];
        uint2 s8 = make_uint2(0, 0);
        uint16_t dbits = 0;
        if (valid) {
            const uint4 *ql = reinterpret_cast<const uint4 *>(w + pl.off[0] + sb * 128 + 64 * hh + 32 * u);
            const uint4 *qh = reinterpret_cast<const uint4 *>(w + pl.off[1] + sb * 64 + 32 * hh);
            const uint4 L0 = ql[0], L1 = ql[1], H0 = qh[0], H1 = qh[1];
            const uint32_t lw[8] = {L0.x, L0.y, L0.z, L0.w, L1.x, L1.y, L1.z, L1.w};
            const uint32_t hw[8] = {H0.x, H0.y, H0.z, H0.w, H1.x, H1.y, H1.z, H1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                lo[i] = (lw[i] & 0x0F0F0F0Fu) | (((hw[i] >> (2 * u)) & 0x03030303u) << 4);
                hi[i] = ((lw[i] >> 4) & 0x0F0F0F0Fu) | (((hw[i] >> (2 * u + 4)) & 0x03030303u) << 4);
            }
            s8 = *reinterpret_cast<const uint2 *>(w + pl.off[2] + sb * 16 + 8 * hh);
            dbits = *reinterpret_cast<const uint16_t *>(w + pl.off[3] + sb * 2);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) lo[i] = hi[i] = 0x20202020u;  // q = 32: w' = 0
        }
        const int sa = (int8_t)byte_of(s8.x, 2 * u), sb_ = (int8_t)byte_of(s8.x, 2 * u + 1);
        const int sc_ = (int8_t)byte_of(s8.y, 2 * u), sd = (int8_t)byte_of(s8.y, 2 * u + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            digits_q6(lo[i], sa, h0[i], l0[i]);
            digits_q6(lo[i + 4], sb_, h0[i + 4], l0[i + 4]);
            digits_q6(hi[i], sc_, h1[i], l1[i]);
            digits_q6(hi[i + 4], sd, h1[i + 4], l1[i + 4]);
        }
        const int k0 = 128 * hh + 32 * u;
        store_digits<FMT>(wh, wl, r, k0, h0, l0);
        store_digits<FMT>(wh, wl, r, k0 + 64, h1, l1);
        if (c == 0) {
            dn[r] = valid ? f16_bits_to_float(dbits) : 0.0f;
            dmn[r] = 0.0f;
        }
        return;
    }
    uint4 h = make_uint4(0, 0, 0, 0), q0 = h, q1 = h, hb0 = h, hb1 = h;
    if (valid) {
        h = *reinterpret_cast<const uint4 *>(w + pl.off[0] + sb * 16);
        const int64_t qs_off = FMT == KQ_Q4_K ? pl.off[1] : pl.off[2];
        const uint4 *qs = reinterpret_cast<const uint4 *>(w + qs_off + sb * 128 + 32 * c);
        q0 = qs[0];
        q1 = qs[1];
        if (FMT == KQ_Q5_K) {
            const uint4 *qh = reinterpret_cast<const uint4 *>(w + pl.off[1] + sb * 32);
            hb0 = qh[0];
            hb1 = qh[1];
        }
    }
    uint32_t lo[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    const uint32_t hb[8] = {hb0.x, hb0.y, hb0.z, hb0.w, hb1.x, hb1.y, hb1.z, hb1.w};
    uint32_t hi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        hi[i] = (lo[i] >> 4) & 0x0F0F0F0Fu;
        lo[i] &= 0x0F0F0F0Fu;
        if (FMT == KQ_Q5_K) {
            lo[i] |= ((hb[i] >> (2 * c)) & 0x01010101u) << 4;
            hi[i] |= ((hb[i] >> (2 * c + 1)) & 0x01010101u) << 4;
        }
    }
    int sc0, m0, sc1, m1;
    scale_min_6bit(h.y, h.z, h.w, 2 * c, sc0, m0);
    scale_min_6bit(h.y, h.z, h.w, 2 * c + 1, sc1, m1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        digits_q45(lo[i], sc0, h0[i], l0[i]);
        digits_q45(hi[i], sc1, h1[i], l1[i]);
    }
    store_digits<FMT>(wh, wl, r, 64 * c, h0, l0);
    store_digits<FMT>(wh, wl, r, 64 * c + 32, h1, l1);
    // min of sub-block j pairs with bsums 2j and 2j+1
    _Float16 *me = mexp + r * 16 + 4 * c;
    me[0] = me[1] = (_Float16)m0;
    me[2] = me[3] = (_Float16)m1;
    if (c == 0) {
        dn[r] = f16_bits_to_float(h.x & 0xFFFFu);
        dmn[r] = f16_bits_to_float(h.x >> 16);
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

template <int FMT, int WM, int TN, bool PART>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t *__restrict__ w, int64_t n, int nsb,
                                                   const int8_t *__restrict__ xq, const float *__restrict__ xs,
                                                   const int16_t *__restrict__ xbs, int64_t mtok,
                                                   float *__restrict__ y, int32_t *__restrict__ Pout,
                                                   int32_t *__restrict__ Mout, int mtiles)
{
    constexpr int WN = 4 / WM;
    constexpr int BM = 64 * WM, BN = 32 * TN * WN;
    __shared__ __align__(16) int8_t wh[BN * LDS_STRIDE];
    __shared__ __align__(16) int8_t wl[BN * LDS_STRIDE];
    __shared__ __align__(16) _Float16 mexp[BN * 16];
    __shared__ float dn[BN], dmn[BN];
    __shared__ __align__(16) float d8s[BM];

    int nt, mt;
    tile_of(blockIdx.x, gridDim.x, mtiles, nt, mt);
    const int64_t n0 = (int64_t)nt * BN, m0 = (int64_t)mt * BM;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int l32 = lane & 31, lh = lane >> 5;
    const int64_t K = (int64_t)nsb * QK, KB = K / 16;
    const Planes pl = planes_of(FMT, n, nsb);

    f32x16 accf[2][TN];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) accf[mi][ni] = f32x16{};

    for (int s = 0; s < nsb; ++s) {
        __syncthreads();  // the previous superblock's panel is consumed
        for (int task = threadIdx.x; task < BN * 4; task += 256) {
            const int r = task >> 2, c = task & 3;
            const int64_t row = n0 + r;
            const bool valid = row < n;
            unpack_task<FMT>(w, pl, valid ? row * nsb + s : 0, valid, r, c, wh, wl, mexp, dn, dmn);
        }
        for (int i = threadIdx.x; i < BM; i += 256) {
            const int64_t t = m0 + i;
            d8s[i] = t < mtok ? xs[t * nsb + s] : 0.0f;
        }
        // A operands (Q8_K codes) and the bsums of this superblock
        i32x4 A[2][8];
        f16x8 Ab[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            const int64_t t = m0 + wm * 64 + mi * 32 + l32;
            const bool tv = t < mtok;
            const int8_t *ap = xq + (tv ? t : 0) * K + (int64_t)s * QK + 16 * lh;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) A[mi][ks] = tv ? *reinterpret_cast<const i32x4 *>(ap + 32 * ks) : i32x4{};
            const uint4 b = tv ? *reinterpret_cast<const uint4 *>(xbs + t * KB + (int64_t)s * 16 + 8 * lh)
                               : make_uint4(0, 0, 0, 0);
            const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Ab[mi][2 * e] = (_Float16)(int16_t)(bw[e] & 0xFFFF);
                Ab[mi][2 * e + 1] = (_Float16)(int16_t)(bw[e] >> 16);
            }
        }
        __syncthreads();  // the panel is complete

        i32x16 acci[2][TN];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < TN; ++ni) acci[mi][ni] = i32x16{};
        // high-digit pass
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int ni = 0; ni < TN; ++ni) {
                const int rl = wn * 32 * TN + ni * 32 + l32;
                const i32x4 B = *reinterpret_cast<const i32x4 *>(wh + rl * LDS_STRIDE + 32 * ks + 16 * lh);
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
                    acci[mi][ni] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[mi][ks], B, acci[mi][ni], 0, 0, 0);
            }
        }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < TN; ++ni) acci[mi][ni] = acci[mi][ni] * 128;
        // low-digit pass
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int ni = 0; ni < TN; ++ni) {
                const int rl = wn * 32 * TN + ni * 32 + l32;
                const i32x4 B = *reinterpret_cast<const i32x4 *>(wl + rl * LDS_STRIDE + 32 * ks + 16 * lh);
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
                    acci[mi][ni] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[mi][ks], B, acci[mi][ni], 0, 0, 0);
            }
        }
        // min term and the per-superblock float fold
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) {
            const int rl = wn * 32 * TN + ni * 32 + l32;
            const float dv = dn[rl], dm = dmn[rl];
            f16x8 Bm{};
            if (FMT != KQ_Q6_K) Bm = *reinterpret_cast<const f16x8 *>(mexp + rl * 16 + 8 * lh);
            const int64_t col = n0 + rl;
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                f32x16 mf{};
                if (FMT != KQ_Q6_K) mf = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ab[mi], Bm, mf, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int tl = wm * 64 + mi * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
                    const float Pf = (float)acci[mi][ni][i];
                    const float u = FMT == KQ_Q6_K ? dv * Pf : fmaf(dv, Pf, -(dm * mf[i]));
                    accf[mi][ni][i] = fmaf(d8s[tl], u, accf[mi][ni][i]);
                    if (PART) {
                        const int64_t t = m0 + tl;
                        if (t < mtok && col < n) {
                            const int64_t o = (t * n + col) * nsb + s;
                            Pout[o] = acci[mi][ni][i];
                            if (Mout) Mout[o] = FMT == KQ_Q6_K ? 0 : (int)mf[i];
                        }
                    }
                }
            }
        }
    }

#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) {
            const int64_t col = n0 + wn * 32 * TN + ni * 32 + l32;
            if (col >= n) continue;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int64_t t = m0 + wm * 64 + mi * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
                if (t < mtok) y[t * n + col] = accf[mi][ni][i];
            }
        }
}

template <int FMT, int WM, int TN>
static void launch_cfg(bool part, int64_t n, int nsb, const uint8_t *w, const int8_t *xq, const float *xs,
                       const int16_t *xbs, int64_t m, float *y, int32_t *P, int32_t *M, hipStream_t st)
{
    constexpr int WN = 4 / WM;
    constexpr int BM = 64 * WM, BN = 32 * TN * WN;
    const int64_t ntiles = (n + BN - 1) / BN, mtiles = (m + BM - 1) / BM;
    const dim3 g((unsigned)(ntiles * mtiles)), b(256);
    if (part)
        hipLaunchKernelGGL((gemm_kernel<FMT, WM, TN, true>), g, b, 0, st, w, n, nsb, xq, xs, xbs, m, y, P, M,
                           (int)mtiles);
    else
        hipLaunchKernelGGL((gemm_kernel<FMT, WM, TN, false>), g, b, 0, st, w, n, nsb, xq, xs, xbs, m, y, P, M,
                           (int)mtiles);
}

template <int FMT>
static void launch_fmt(bool part, int64_t n, int nsb, const uint8_t *w, const int8_t *xq, const float *xs,
                       const int16_t *xbs, int64_t m, float *y, int32_t *P, int32_t *M, hipStream_t st)
{
    // 256 x 64 tiles when that fills the chip, else 256 x 32
    const int64_t tiles_64 = ((n + 63) / 64) * ((m + 255) / 256);
    if (tiles_64 >= 256)
        launch_cfg<FMT, 4, 2>(part, n, nsb, w, xq, xs, xbs, m, y, P, M, st);
    else
        launch_cfg<FMT, 4, 1>(part, n, nsb, w, xq, xs, xbs, m, y, P, M, st);
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
