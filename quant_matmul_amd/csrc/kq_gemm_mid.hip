// kq_gemm_mid.hip -- the K-quant x Q8_K matmul for token counts between the
// GEMV and the prefill tile (9..127 tokens), and the grouped form that runs
// every expert of a mixture-of-experts layer in one launch.
//
// Same integer partials and float fold as kq_gemm (K-quant kernel arc page,
// "The pieces", kq v2 item), the min term on v_mfma_f32_32x32x16_f16.  What
// changes is where and how the weights are unpacked.  With 32 tokens per
// tile the unpack, not the matrix cores, bounds the kernel, and a shared
// LDS panel would only add traffic and barriers: each lane unpacks its own
// half superblock row (128 weights) straight into MFMA B-operand registers.
// A wave owns 32 weight rows x 32 tokens; its lane l holds row l%32 and the
// codes k = 32*ks + 16*(l/32) + 0..15 of each 32-deep K step ks, which is
// exactly the B operand of v_mfma_i32_32x32x32_i8.
//  * Q4_K/Q5_K: a 32-weight sub-block is one K step, so the raw quants go to
//    the MFMA as they are and its output is dot_j; the sub-scale is one
//    integer mad per output, P += sc_j * dot_j.  At 32 tokens that costs
//    less than folding sc_j into two digit planes (the prefill tile's
//    choice, which pays off when 256 tokens share each unpacked weight).
//  * Q6_K: 16-weight sub-blocks do not match a K step, so it keeps the
//    digit passes (kq_digits.h), high and low digit in two accumulators.
// Waves share nothing but L2: no barriers.  The page's mid-size lesson (the chain-regrain / nrsplit
// commits: splitting tokens re-ran the unpack per slice) is why a tile
// covers its 32 tokens in one pass and the grid splits rows and, when the
// grid is small, K -- never tokens.
//
// Grouped form: the activation rows are gathered per expert into one tile
// image, each expert's rows padded to whole 32-row tiles, and tile_expert
// names the expert of every 32-row tile; its weights are the planes at
// w_planes + expert * w_stride.  The page's MoE path fills one Q8_K image
// for the gate and up projections ("The pieces", kq v2 item).
#include "kq_common.h"
#include "kq_digits.h"

namespace kq {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

namespace {

// Raw bytes of one lane's half superblock row (lane half lh takes the codes
// k = 32*ks + 16*lh + e of every K step ks):
//  Q4_K/Q5_K: weights 64c + 16lh + e and 64c + 32 + 16lh + e are the low
//    and high nibbles of quant byte 32c + 16lh + e; Q5_K's fifth bit of
//    sub-block j is bit j of high-bit byte 16lh + e.
//  Q6_K: weight 128h + 32u + 16lh + e takes nibble u/2 of low byte
//    64h + 32(u%2) + 16lh + e and bits 2u, 2u+1 of high byte 32h + 16lh + e;
//    its scale is that of 16-weight sub-block 8h + 2u + lh.
template <int FMT>
struct Lane;
template <>
struct Lane<KQ_Q4_K> {
    uint4 h, q[4];
};
template <>
struct Lane<KQ_Q5_K> {
    uint4 h, q[4], qh;
};
template <>
struct Lane<KQ_Q6_K> {
    uint4 l[4], hq[2], sc;
    uint32_t d;
};

__device__ inline void load_lane(Lane<KQ_Q4_K> &r, const uint8_t *__restrict__ w, const Planes &pl, int64_t sb,
                                 int lh)
{
    r.h = *reinterpret_cast<const uint4 *>(w + pl.off[0] + sb * 16);
#pragma unroll
    for (int c = 0; c < 4; ++c) r.q[c] = *reinterpret_cast<const uint4 *>(w + pl.off[1] + sb * 128 + 32 * c + 16 * lh);
}
__device__ inline void load_lane(Lane<KQ_Q5_K> &r, const uint8_t *__restrict__ w, const Planes &pl, int64_t sb,
                                 int lh)
{
    r.h = *reinterpret_cast<const uint4 *>(w + pl.off[0] + sb * 16);
    r.qh = *reinterpret_cast<const uint4 *>(w + pl.off[1] + sb * 32 + 16 * lh);
#pragma unroll
    for (int c = 0; c < 4; ++c) r.q[c] = *reinterpret_cast<const uint4 *>(w + pl.off[2] + sb * 128 + 32 * c + 16 * lh);
}
__device__ inline void load_lane(Lane<KQ_Q6_K> &r, const uint8_t *__restrict__ w, const Planes &pl, int64_t sb,
                                 int lh)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r.l[i] = *reinterpret_cast<const uint4 *>(w + pl.off[0] + sb * 128 + 32 * i + 16 * lh);
#pragma unroll
    for (int h = 0; h < 2; ++h) r.hq[h] = *reinterpret_cast<const uint4 *>(w + pl.off[1] + sb * 64 + 32 * h + 16 * lh);
    r.sc = *reinterpret_cast<const uint4 *>(w + pl.off[2] + sb * 16);
    r.d = *reinterpret_cast<const uint16_t *>(w + pl.off[3] + sb * 2);
}

__device__ inline uint32_t word(const uint4 &v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

// Q6_K digits (B operands) of K step ks of the lane's half row
template <int FMT>
__device__ inline void digits_ks(const Lane<FMT> &r, int ks, int lh, i32x4 &bh, i32x4 &bl)
{
    uint32_t h[4], l[4];
    if constexpr (FMT == KQ_Q6_K) {
        const int hh = ks >> 2, u = ks & 3;
        const int sc = (int8_t)byte_of(word(r.sc, (2 * ks + lh) >> 2), (2 * ks + lh) & 3);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lw = word(r.l[2 * hh + (u & 1)], i);
            const uint32_t nib = (u >> 1) ? (lw >> 4) & 0x0F0F0F0Fu : lw & 0x0F0F0F0Fu;
            const uint32_t q = nib | (((word(r.hq[hh], i) >> (2 * u)) & 0x03030303u) << 4);
            digits_q6(q, sc, h[i], l[i]);
        }
    } else {
        const int c = ks >> 1;
        int sc, m;
        scale_min_6bit(r.h.y, r.h.z, r.h.w, ks, sc, m);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t qw = word(r.q[c], i);
            uint32_t q = (ks & 1) ? (qw >> 4) & 0x0F0F0F0Fu : qw & 0x0F0F0F0Fu;
            if constexpr (FMT == KQ_Q5_K) q |= ((word(r.qh, i) >> ks) & 0x01010101u) << 4;
            digits_q45(q, sc, h[i], l[i]);
        }
    }
    bh = i32x4{(int)h[0], (int)h[1], (int)h[2], (int)h[3]};
    bl = i32x4{(int)l[0], (int)l[1], (int)l[2], (int)l[3]};
}

__device__ inline int item_of_mid(int b, int G)
{
    const int per = G / 8;
    return b < per * 8 ? (b % 8) * per + b / 8 : b;
}

}  // namespace

template <int FMT, bool GROUPED, bool PART>
__global__ __launch_bounds__(256, 2) void gemm_mid_kernel(
    const uint8_t *__restrict__ w, int64_t w_stride, const int32_t *__restrict__ tile_expert, int experts, int64_t n,
    int nsb, const int8_t *__restrict__ xq, const float *__restrict__ xs, const _Float16 *__restrict__ xbs,
    int64_t mtok, float *__restrict__ y, int32_t *__restrict__ Pout, int32_t *__restrict__ Mout, int mtiles, int S)
{
    __shared__ __align__(16) float d8w[4][32];

    // item = (128-row panel, 32-token tile, K split): the token tiles of a
    // panel run on one XCD and share its L2 copy of the panel's planes
    const int item = item_of_mid(blockIdx.x, gridDim.x);
    const int tile = item / S, split = item - tile * S;
    const int nt = tile / mtiles, mt = tile - nt * mtiles;
    const int s0 = (int)((int64_t)nsb * split / S), s1 = (int)((int64_t)nsb * (split + 1) / S);
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
    const int64_t row0 = (int64_t)nt * 128 + wv * 32;
    if (row0 >= n) return;  // whole wave: no rows of its own
    const int64_t row = row0 + lr;
    const bool rvalid = row < n;
    const int64_t m0 = (int64_t)mt * 32;
    const uint8_t *wb = w;
    if constexpr (GROUPED) {
        const int e = tile_expert[mt];
        if (e < 0 || e >= experts) return;  // no such expert: tile left unwritten
        wb += (int64_t)e * w_stride;
    }
    const int64_t K = (int64_t)nsb * QK;
    const Planes pl = planes_of(FMT, n, nsb);
    const int64_t wrow = (rvalid ? row : n - 1) * nsb;

    // the tile's 32 tokens of codes and f16 bsums (tile image) and d8s
    const int64_t mpad = (mtok + 31) & ~(int64_t)31;
    const uint64_t a_bytes = (uint64_t)(mpad - m0) * (uint64_t)K;
    const uint64_t b_bytes = (uint64_t)(mpad - m0) * (uint64_t)nsb * 32;
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xq + m0 * K), 0, (int)(uint32_t)(a_bytes < 0xFFFFFFFFu ? a_bytes : 0xFFFFFFFFu), 0x00020000);
    const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xbs + m0 * nsb * 16), 0, (int)(uint32_t)(b_bytes < 0xFFFFFFFFu ? b_bytes : 0xFFFFFFFFu),
        0x00020000);
    const int64_t td = m0 + lr;  // token whose d8 this lane stages
    const float *xs_row = xs + (td < mtok ? td : mtok - 1) * nsb;

    i32x4 A[8];
    f16x8 Ab;
    Lane<FMT> raw, nxt;
    float d8v;
    auto load_a = [&](int s, int ks) {
        A[ks] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, (s * 8 + ks) * 1024 + 16 * lane, 0, 0));
    };
    auto load_bs = [&](int s) {
        if constexpr (FMT != KQ_Q6_K)
            Ab = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(rB, s * 1024 + 16 * lane, 0, 0));
    };

    f32x16 accf = f32x16{};
    load_lane(raw, wb, pl, wrow + s0, lh);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) load_a(s0, ks);
    load_bs(s0);
    d8v = td < mtok ? xs_row[s0] : 0.0f;

    for (int s = s0; s < s1; ++s) {
        // operands of the next superblock are fetched unconditionally (the
        // last step re-reads its own, in bounds): a branch here would split
        // the K loop into blocks the scheduler cannot interleave across
        const int sn = s + 1 < s1 ? s + 1 : s;
        // stage the 32 d8s of superblock s for the fold (wave-private LDS:
        // the wave's own later reads see these writes in order)
        if (lh == 0) d8w[wv][lr] = d8v;
        load_lane(nxt, wb, pl, wrow + sn, lh);
        d8v = td < mtok ? xs_row[sn] : 0.0f;
        float dv, dm = 0.0f;
        f32x16 mf;
        i32x16 P;
        if constexpr (FMT == KQ_Q6_K) {
            // 16-weight sub-blocks: the scale is folded into the two digit
            // passes (kq_digits.h)
            i32x16 acch = i32x16{}, accl = i32x16{};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                i32x4 bh, bl;
                digits_ks<FMT>(raw, ks, lh, bh, bl);
                acch = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[ks], bh, acch, 0, 0, 0);
                accl = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[ks], bl, accl, 0, 0, 0);
                load_a(sn, ks);
            }
            P = (acch << 7) + accl;
            dv = rvalid ? f16_bits_to_float(raw.d) : 0.0f;
        } else {
            // 32-weight sub-blocks = one 32-deep K step: the raw quants are
            // the B operand, dot_j comes out of one MFMA and the sub-scale is
            // applied with one 24-bit integer mad per output (|dot_j| <=
            // 31*127*32 < 2^23, |P| < 2^26): P = sum_j sc_j * dot_j exactly
            const uint32_t s0w = raw.h.y, s1w = raw.h.z, s2w = raw.h.w;
            // the eight 6-bit scales and mins, four per word, as bytes
            const uint32_t sc_lo = s0w & 0x3F3F3F3Fu;
            const uint32_t sc_hi = (s2w & 0x0F0F0F0Fu) | ((s0w >> 2) & 0x30303030u);
            const uint32_t m_lo = s1w & 0x3F3F3F3Fu;
            const uint32_t m_hi = ((s2w >> 4) & 0x0F0F0F0Fu) | ((s1w >> 2) & 0x30303030u);
            P = i32x16{};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                i32x4 bq;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t qw = word(raw.q[ks >> 1], i);
                    uint32_t q = (ks & 1) ? (qw >> 4) & 0x0F0F0F0Fu : qw & 0x0F0F0F0Fu;
                    if constexpr (FMT == KQ_Q5_K) q |= ((word(raw.qh, i) >> ks) & 0x01010101u) << 4;
                    bq[i] = (int)q;
                }
                const i32x16 d = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[ks], bq, i32x16{}, 0, 0, 0);
                const int sc = (int)byte_of(ks < 4 ? sc_lo : sc_hi, ks & 3);
#pragma unroll
                for (int i = 0; i < 16; ++i) P[i] = __mul24(d[i], sc) + P[i];
                load_a(sn, ks);
            }
            dv = rvalid ? f16_bits_to_float(raw.h.x & 0xFFFFu) : 0.0f;
            dm = rvalid ? f16_bits_to_float(raw.h.x >> 16) : 0.0f;
            // min term: B operand = m of the sub-block of bsums 8lh + 0..7
            const uint32_t mw = lh ? m_hi : m_lo;
            f16x8 bm;
#pragma unroll
            for (int j = 0; j < 4; ++j) bm[2 * j] = bm[2 * j + 1] = (_Float16)(int)byte_of(mw, j);
            mf = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ab, bm, f32x16{}, 0, 0, 0);
            load_bs(sn);
        }
        __builtin_amdgcn_wave_barrier();
        // lane holds tokens 8*(i/4) + 4*lh + i%4, i = 0..15, of row `row`
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int tl = 8 * (i >> 2) + 4 * lh + (i & 3);
            const float Pf = (float)P[i];
            float u;
            if constexpr (FMT == KQ_Q6_K) u = dv * Pf;
            else u = fmaf(dv, Pf, -(dm * mf[i]));
            accf[i] = fmaf(d8w[wv][tl], u, accf[i]);
            if (PART) {
                const int64_t t = m0 + tl;
                if (t < mtok && rvalid) {
                    const int64_t o = (t * n + row) * nsb + s;
                    Pout[o] = P[i];
                    if (Mout) {
                        if constexpr (FMT == KQ_Q6_K) Mout[o] = 0;
                        else Mout[o] = (int)mf[i];
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        raw = nxt;
    }

    // K split j of S writes slice j of y (y then points at the workspace)
    if (!rvalid) return;
    float *yo = y + (int64_t)split * mtok * n;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t t = m0 + 8 * (i >> 2) + 4 * lh + (i & 3);
        if (t < mtok) yo[t * n + row] = accf[i];
    }
}

void launch_sum_splits(const float *p, int S, int64_t count, float *y, hipStream_t st);

namespace {

int pick_splits_mid(int64_t waves, int nsb)
{
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 256;
    }
    // about 8 resident waves per CU
    int S = (int)((8 * (int64_t)cus) / waves);
    S = S < nsb / 2 ? S : nsb / 2;
    S = S < 8 ? S : 8;
    return S > 1 ? S : 1;
}

template <int FMT, bool GROUPED>
void launch_mid_fmt(bool part, const uint8_t *w, int64_t w_stride, const int32_t *tile_expert, int experts,
                    int64_t n, int nsb, const int8_t *xq, const float *xs, const _Float16 *xbs, int64_t m, float *y,
                    int32_t *P, int32_t *M, int S, hipStream_t st)
{
    const int64_t ntiles = (n + 127) / 128, mtiles = (m + 31) / 32;
    const dim3 g((unsigned)(ntiles * mtiles * S)), b(256);
    if (part)
        hipLaunchKernelGGL((gemm_mid_kernel<FMT, GROUPED, true>), g, b, 0, st, w, w_stride, tile_expert, experts, n,
                           nsb, xq, xs, xbs, m, y, P, M, (int)mtiles, S);
    else
        hipLaunchKernelGGL((gemm_mid_kernel<FMT, GROUPED, false>), g, b, 0, st, w, w_stride, tile_expert, experts, n,
                           nsb, xq, xs, xbs, m, y, P, M, (int)mtiles, S);
}

template <bool GROUPED>
void launch_mid_any(int fmt, bool part, const uint8_t *w, int64_t w_stride, const int32_t *tile_expert, int experts,
                    int64_t n, int nsb, const int8_t *xq, const float *xs, const _Float16 *xbs, int64_t m, float *y,
                    int32_t *P, int32_t *M, int S, hipStream_t st)
{
    if (fmt == KQ_Q4_K)
        launch_mid_fmt<KQ_Q4_K, GROUPED>(part, w, w_stride, tile_expert, experts, n, nsb, xq, xs, xbs, m, y, P, M, S,
                                         st);
    else if (fmt == KQ_Q5_K)
        launch_mid_fmt<KQ_Q5_K, GROUPED>(part, w, w_stride, tile_expert, experts, n, nsb, xq, xs, xbs, m, y, P, M, S,
                                         st);
    else
        launch_mid_fmt<KQ_Q6_K, GROUPED>(part, w, w_stride, tile_expert, experts, n, nsb, xq, xs, xbs, m, y, P, M, S,
                                         st);
}

int64_t mid_waves(int64_t n, int64_t m) { return ((n + 31) / 32) * ((m + 31) / 32); }

}  // namespace

size_t gemm_mid_workspace_bytes(int64_t n, int64_t k, int64_t m)
{
    const int S = pick_splits_mid(mid_waves(n, m), (int)(k / QK));
    return S == 1 ? 0 : (size_t)S * (size_t)m * (size_t)n * 4;
}

int launch_gemm_mid(int fmt, const void *w, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                    const void *xbs, int64_t m, float *y, int32_t *P, int32_t *M, void *ws, size_t ws_bytes,
                    hipStream_t st)
{
    const int nsb = (int)(k / QK);
    const bool part = P != nullptr;
    int S = 1;
    if (!part && ws && ws_bytes >= gemm_mid_workspace_bytes(n, k, m)) S = pick_splits_mid(mid_waves(n, m), nsb);
    float *dst = S > 1 ? (float *)ws : y;
    launch_mid_any<false>(fmt, part, (const uint8_t *)w, 0, nullptr, 0, n, nsb, xq, xs, (const _Float16 *)xbs, m, dst,
                          P, M, S, st);
    if (S > 1) launch_sum_splits((const float *)ws, S, m * n, y, st);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ELAUNCH;
}

int launch_gemm_grouped(int fmt, const void *w, int64_t w_stride, int64_t experts, const int32_t *tile_expert,
                        int64_t n, int64_t k, const int8_t *xq, const float *xs, const void *xbs, int64_t m,
                        float *y, int32_t *P, int32_t *M, hipStream_t st)
{
    launch_mid_any<true>(fmt, P != nullptr, (const uint8_t *)w, w_stride, tile_expert, (int)experts, n,
                         (int)(k / QK), xq, xs, (const _Float16 *)xbs, m, y, P, M, 1, st);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ELAUNCH;
}

}  // namespace kq
