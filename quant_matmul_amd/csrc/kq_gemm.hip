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
//    raw quant but the sub-scale-folded weight w' = sc*q (Q4_K/Q5_K) or
//    sc*(q-32) (Q6_K, -4064..4096) as two int8 digits (kq_digits.h): the
//    MFMA cannot apply a per-row, per-sub-block scale, so folding it into
//    the operand is what keeps the per-sub-block integer fold on the matrix
//    cores.  Q5_K/Q6_K use w' = 128*h + l; Q4_K, whose quants are 4-bit,
//    splits the scale instead (sc = 8u + v, digits u*q and v*q), which one
//    packed 16-bit multiply forms four at a time.
//  * Dense contraction: v_mfma_i32_32x32x32_i8, a high-digit pass, a shift
//    by 7 (Q4_K: 3), a low-digit pass into the same int32 accumulator --
//    which then holds P = sum_j sc_j * dot_j exactly (|P| < 2^27).  The
//    32x32x32 form sustains about twice the int8 rate of the 16x16x64 form
//    on gfx950.
//  * Min term: M = sum_g m_{g/2} * bsum_g is a 16-deep contraction per
//    superblock, one v_mfma_f32_32x32x16_f16 (bsums |.| <= 2032 and m <= 63
//    are exact in f16, and |M| < 2^24 keeps the f32 sum exact).
//  * Epilogue per superblock: acc += d8 * (d*P - dmin*M).
//
// Operands from HBM.  The codes and the f16 bsums come from the tile image
// of the Q8_K quantiser (32 tokens per 1 KiB operand), so each A operand is
// one coalesced 1 KiB load with no conversion; row-major codes spread it
// over 32 partly used cache lines, and that L2-to-L1 traffic, not the
// matrix cores, bounded the kernel.  Both are read through buffer resources
// based at the workgroup's first token: tokens past the image read as zero
// and their outputs are never stored.
//
// Pipeline.  A workgroup is 4 waves over a 256-token x 32-row tile; each
// wave owns 64 tokens x 32 rows (two 32x32 MFMA tiles).  Per superblock s
// the wave's codes sit in registers, the digit panel in one of two LDS
// buffers; while the high-digit MFMAs of s run, the wave unpacks its share
// of superblock s+1 (whose packed bytes were prefetched) into the other
// buffer, so the VALU unpack overlaps the matrix pipe; the low-digit passes
// of the two tiles are interleaved, so two independent MFMA chains are in
// flight there too (run tile by tile, each a single dependent chain, the
// pass was 4-6% slower over the whole kernel even with tile 0's fold under
// tile 1's MFMAs); each 32-deep K step of the codes is refilled with
// superblock s+1 as soon as it is dead.  The loop body is one basic block (no divergent
// branch: validity is masked, every refill is unconditional), so the
// scheduler can interleave all of it.  One barrier per superblock.
#include <atomic>

#include "kq_common.h"
#include "kq_digits.h"

namespace kq {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int LDS_STRIDE = 272;  // bytes per digit row: 256 + 16 pad

namespace {

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
    const uint32_t vm = valid ? 0xFFFFFFFFu : 0u;
    const uint2 s8 = make_uint2(rw.s8.x & vm, rw.s8.y & vm);
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
    // every task of the row writes the same scale (no divergent branch)
    dn[r] = valid ? f16_bits_to_float(rw.d) : 0.0f;
    dmn[r] = 0.0f;
}

template <int FMT>
__device__ inline void unpack_half(const Half<FMT> &rw, bool valid, int r, int h, int8_t *wh, int8_t *wl,
                                   _Float16 *mexp, float *dn, float *dmn)
{
    const int c = h >> 1, half = h & 1;
    // rows past n: scales and mins masked to zero (an AND, not a branch)
    const uint32_t vm = valid ? 0xFFFFFFFFu : 0u;
    const uint4 hd = make_uint4(rw.h.x & vm, rw.h.y & vm, rw.h.z & vm, rw.h.w & vm);
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
            digits_q45(lo, sc0, h0[i], l0[i]);
            digits_q45(hi, sc1, h1[i], l1[i]);
        } else {
            digits_q4(lo, sc0 >> 3, sc0 & 7, h0[i], l0[i]);
            digits_q4(hi, sc1 >> 3, sc1 & 7, h1[i], l1[i]);
        }
    }
    const int k0 = 64 * c + 16 * half;
    store_half(wh, wl, r, k0, h0, l0);
    store_half(wh, wl, r, k0 + 32, h1, l1);
    // min of sub-block j pairs with bsums 2j and 2j+1: the half-0 task
    // writes sub-block 2c's pair, the half-1 task 2c+1's; every task of the
    // row writes the same d, dmin (no divergent branch)
    const _Float16 mv = (_Float16)(half ? m1 : m0);
    *reinterpret_cast<f16x2 *>(mexp + r * 16 + 4 * c + 2 * half) = f16x2{mv, mv};
    dn[r] = f16_bits_to_float(hd.x & 0xFFFFu);
    dmn[r] = f16_bits_to_float(hd.x >> 16);
}

// Workgroup index -> work item, grouping consecutive items on one XCD
// (workgroup b runs on XCD b % 8).  Items are ordered (row panel, token
// block, K split), so the token blocks of one row panel share that XCD's
// L2 copy of the panel's packed planes.
__device__ inline int item_of(int b, int G)
{
    const int per = G / 8;
    return b < per * 8 ? (b % 8) * per + b / 8 : b;
}

}  // namespace

// Two workgroups per CU.  The partials form (PART: every superblock's P and M
// stored too) holds one, so its extra live values sit in the accumulation
// registers instead of spilling to scratch; the arithmetic is the same.
template <int FMT, bool PART>
__global__ __launch_bounds__(256, PART ? 1 : 2) void gemm_kernel(const uint8_t *__restrict__ w, int64_t n, int nsb,
                                                      const int8_t *__restrict__ xq, const float *__restrict__ xs,
                                                      const _Float16 *__restrict__ xbs, int64_t mtok,
                                                      float *__restrict__ y, int32_t *__restrict__ Pout,
                                                      int32_t *__restrict__ Mout, int mtiles, int full, int TS,
                                                      float *__restrict__ ws, unsigned long long *__restrict__ cnt,
                                                      unsigned long long seq)
{
    constexpr int BM = 256, BN = 32;
    static_assert(BN * 8 == 256, "one 32-weight unpack task per thread");
    __shared__ __align__(16) int8_t wh[2][BN * LDS_STRIDE];
    __shared__ __align__(16) int8_t wl[2][BN * LDS_STRIDE];
    __shared__ __align__(16) _Float16 mexp[2][BN * 16];
    __shared__ float dn[2][BN], dmn[2][BN];
    __shared__ __align__(16) float d8s[2][BM];

    // Workgroups 0..full-1 each run one whole tile and write y; the rest run
    // the remaining tiles split along K in TS parts (split j covers
    // superblocks [s0, s1)) and write partial tiles to ws; the last part of
    // a tile to finish adds them up.  The whole tiles come first in dispatch
    // order, so split ones would fill the tail (the plan splits only grids
    // smaller than one round, so full is 0 whenever TS > 1).
    int tile, split = 0, S = 1;
    if ((int)blockIdx.x < full) {
        tile = item_of(blockIdx.x, full);
    } else {
        const int r = item_of(blockIdx.x - full, gridDim.x - full);
        tile = full + r / TS;
        split = r - (r / TS) * TS;
        S = TS;
    }
    const int nt = tile / mtiles, mt = tile - nt * mtiles;
    const int s0 = (int)((int64_t)nsb * split / S), s1 = (int)((int64_t)nsb * (split + 1) / S);
    const int64_t n0 = (int64_t)nt * BN, m0 = (int64_t)mt * BM;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wm = tid >> 6;
    const int l32 = lane & 31, lh = lane >> 5;
    const int64_t K = (int64_t)nsb * QK;
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
        // unconditional load (xs_row is clamped in bounds), then select
        const float d8v = xs_row[s];
        d8n = t_d8 < mtok ? d8v : 0.0f;
    };
    auto unpack_w = [&](int b) {
        unpack_half(raw, wvalid, tid >> 3, tid & 7, wh[b], wl[b], mexp[b], dn[b], dmn[b]);
        d8s[b][tid] = d8n;
    };

    // Codes (A operand) and f16 bsums (A operand of the min term) of the
    // wave's 64 tokens = two 32-token groups, from the tile image, which
    // holds tokens up to m rounded up to 32.
    const int64_t mpad = (mtok + 31) & ~(int64_t)31;
    const uint64_t a_bytes = (uint64_t)(mpad - m0) * (uint64_t)K;
    const uint64_t b_bytes = (uint64_t)(mpad - m0) * (uint64_t)nsb * 32;
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xq + m0 * K), 0, (int)(uint32_t)(a_bytes < 0xFFFFFFFFu ? a_bytes : 0xFFFFFFFFu), 0x00020000);
    const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xbs + m0 * nsb * 16), 0, (int)(uint32_t)(b_bytes < 0xFFFFFFFFu ? b_bytes : 0xFFFFFFFFu),
        0x00020000);
    // 32-bit offsets: the caller bounds k so that 256 tokens of codes < 2^31
    int aoff[2], boff[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        aoff[mi] = (wm * 2 + mi) * 32 * (int)K + 16 * lane;
        boff[mi] = (wm * 2 + mi) * nsb * 1024 + 16 * lane;
    }
    i32x4 A[2][8];
    f16x8 Ab[2];
    auto load_a = [&](int s, int ks) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
            A[mi][ks] = __builtin_bit_cast(
                i32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, aoff[mi], (s * 8 + ks) * 1024, 0));
    };
    auto load_bs = [&](int s) {
        if constexpr (FMT != KQ_Q6_K) {
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                Ab[mi] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(rB, boff[mi] + s * 1024, 0, 0));
        }
    };

    f32x16 accf[2];
    accf[0] = accf[1] = f32x16{};

    load_w(s0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) load_a(s0, ks);
    load_bs(s0);
    unpack_w(0);
    load_w(s0 + 1 < s1 ? s0 + 1 : s0);
    __syncthreads();

    for (int s = s0; s < s1; ++s) {
        const int b = (s - s0) & 1;
        // the next superblocks' operands are fetched and unpacked
        // unconditionally (clamped to the last one, in bounds, into the free
        // buffer): a branch would split the MFMA loop into blocks the
        // scheduler cannot interleave across
        const int sn = s + 1 < s1 ? s + 1 : s1 - 1, sn2 = s + 2 < s1 ? s + 2 : s1 - 1;
        i32x16 acc[2];
        // high-digit pass (the first K step starts from the zero operand)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const i32x4 B = *reinterpret_cast<const i32x4 *>(wh[b] + l32 * LDS_STRIDE + 32 * ks + 16 * lh);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                acc[mi] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[mi][ks], B, ks == 0 ? i32x16{} : acc[mi], 0, 0, 0);
        }
        // the unpack of the next superblock overlaps these MFMAs
        unpack_w(b ^ 1);
        // weight of the high digit: 8 for Q4_K's sc = 8u + v split, else 128
        constexpr int SHIFT = FMT == KQ_Q4_K ? 3 : 7;
        const float dv = dn[b][l32], dm = dmn[b][l32];
        const int64_t col = n0 + l32;
        f16x8 Bm;
        if constexpr (FMT != KQ_Q6_K) Bm = *reinterpret_cast<const f16x8 *>(mexp[b] + l32 * 16 + 8 * lh);
        f32x16 mf0, mf1;
        if constexpr (FMT != KQ_Q6_K) mf0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ab[0], Bm, f32x16{}, 0, 0, 0);
        // one float fold of superblock s for element r of tile mi; lane l
        // holds row n0 + l%32 and tokens 8*(r/4) + 4*(l/32) + r%4 of each
        // 32-token group
        auto fold = [&](int mi, int r, const f32x16 &mf) {
            const int tl = wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
            const float Pf = (float)acc[mi][r];
            float u;
            if constexpr (FMT == KQ_Q6_K) u = dv * Pf;
            else u = fmaf(dv, Pf, -(dm * mf[r]));
            accf[mi][r] = fmaf(d8s[b][tl], u, accf[mi][r]);
            if (PART) {
                const int64_t t = m0 + tl;
                if (t < mtok && col < n) {
                    const int64_t o = (t * n + col) * nsb + s;
                    Pout[o] = acc[mi][r];
                    if (Mout) {
                        if constexpr (FMT == KQ_Q6_K) Mout[o] = 0;
                        else Mout[o] = (int)mf[r];
                    }
                }
            }
        };
        // low-digit passes of both tiles interleaved (two independent MFMA
        // chains), each K step's codes refilled with superblock s+1 once dead
        acc[0] = acc[0] << SHIFT;
        acc[1] = acc[1] << SHIFT;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const i32x4 B = *reinterpret_cast<const i32x4 *>(wl[b] + l32 * LDS_STRIDE + 32 * ks + 16 * lh);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                acc[mi] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[mi][ks], B, acc[mi], 0, 0, 0);
                A[mi][ks] = __builtin_bit_cast(
                    i32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, aoff[mi], (sn * 8 + ks) * 1024, 0));
            }
        }
        if constexpr (FMT != KQ_Q6_K) mf1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ab[1], Bm, f32x16{}, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) fold(0, r, mf0);
#pragma unroll
        for (int r = 0; r < 16; ++r) fold(1, r, mf1);
        load_bs(sn);
        load_w(sn2);
        __syncthreads();  // panel s+1 complete; panel s free for s+2
    }

    if (S > 1) {
        // Split tile: publish this part (lane-major: element r of tile mi of
        // wave wm at ((wm*32 + mi*16 + r) * 64 + lane)) with agent-scope
        // stores, which write through to memory all XCDs see, wait for them,
        // then count the part in.  The counter word holds (seq << 16 | parts
        // in); a word of another call (any other seq, or garbage) counts as
        // zero, and the last part resets it to (seq, 0) for graph replays of
        // the same call.  No part waits for another: the last to arrive
        // (whichever it is) reads the others back, again at agent scope, so
        // it sees memory rather than a stale line of its own L2, and adds
        // all parts in split order -- deterministic.
        float *part = ws + (int64_t)(tile - full) * S * (BM * BN);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                __hip_atomic_store(part + split * (BM * BN) + ((wm * 32 + mi * 16 + r) << 6) + lane, accf[mi][r],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        __shared__ int last_part;
        if (tid == 0) {
            unsigned long long *c = cnt + (tile - full);
            const unsigned long long tag = seq & 0xFFFFFFFFFFFFull;
            unsigned long long old = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), nv;
            do {  // at most S-1 retries: each failure is another part's success
                const unsigned long long in = (old >> 16) == tag ? (old & 0xFFFF) : 0;
                nv = (tag << 16) | (in + 1);
            } while (!__hip_atomic_compare_exchange_strong(c, &old, nv, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT));
            const bool last = (int)(nv & 0xFFFF) == S;
            if (last) __hip_atomic_store(c, tag << 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last_part = last;
        }
        __syncthreads();
        if (!last_part) return;
        f32x16 sum[2];
        for (int j = 0; j < S; ++j) {
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float v = j == split ? accf[mi][r]
                                               : __hip_atomic_load(part + j * (BM * BN) +
                                                                       ((wm * 32 + mi * 16 + r) << 6) + lane,
                                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    sum[mi][r] = j == 0 ? v : sum[mi][r] + v;
                }
        }
        accf[0] = sum[0];
        accf[1] = sum[1];
    }
    const int64_t col = n0 + l32;
    if (col < n) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t t = m0 + wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (t < mtok) y[t * n + col] = accf[mi][r];
            }
    }
}

// y = ((p_0 + p_1) + p_2) + ... over S whole-output partial slices p_j of
// m*n floats, in split order, one float per thread (y is only 4-byte
// aligned); the K-split form of the 32-token tile (kq_gemm_mid.hip)
__global__ __launch_bounds__(256) void sum_splits(const float *__restrict__ p, int S, int64_t count,
                                                  float *__restrict__ y)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count) return;
    float acc = p[i];
    for (int j = 1; j < S; ++j) acc += p[(int64_t)j * count + i];
    y[i] = acc;
}

void launch_sum_splits(const float *p, int S, int64_t count, float *y, hipStream_t st)
{
    hipLaunchKernelGGL(sum_splits, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st, p, S, count, y);
}

// Grid plan.  `slots` = workgroups resident at once (two per CU at this
// kernel's occupancy).  A grid of at least `slots` tiles runs unsplit.  A
// smaller one (W_down at pp512: 160 tiles) is split along K into up to 8
// parts of at least 3 superblocks so that it fills the chip.  The parts meet
// through the caller's workspace: a small array of counter words, then the
// partial tiles.  A separate summing pass cost more (it re-reads every
// partial from memory in a second launch), and a device-scope fence writes
// back and invalidates the whole L2 of the XCD, so only the partial tiles
// and the counters use coherent (agent-scope) accesses.  Splitting just the
// last, partial round of a larger grid (W_up: 608 tiles on 512 slots) was
// measured too: the parts' fill and hand-over cost what the shorter tail
// saved, so such grids stay unsplit.
struct Plan {
    int full, tail, TS;
};

// the device's CU count, read once (an atomic, so concurrent first calls are
// safe); both GEMM tiles size their grids by it
int cu_count()
{
    static std::atomic<int> cus_once{0};
    int cus = cus_once.load(std::memory_order_relaxed);
    if (!cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 256;
        cus_once.store(cus, std::memory_order_relaxed);
    }
    return cus;
}

static Plan plan_of(int64_t n, int64_t m, int nsb)
{
    const int64_t slots = 2 * (int64_t)cu_count();
    const int64_t tiles = ((n + 31) / 32) * ((m + 255) / 256);
    const int64_t tail = tiles < slots ? tiles : 0;
    Plan p{(int)tiles, 0, 1};
    if (tail == 0) return p;
    int TS = (int)(slots / tail);
    TS = TS < nsb / 3 ? TS : nsb / 3;
    TS = TS < 8 ? TS : 8;
    if (TS < 2) return p;
    return Plan{(int)(tiles - tail), (int)tail, TS};
}

// counter words (one per split tile, 256-byte rounded), then the partials
static size_t counter_bytes(const Plan &p) { return ((size_t)p.tail * 8 + 255) / 256 * 256; }

size_t gemm_workspace_bytes(int64_t n, int64_t k, int64_t m)
{
    const Plan p = plan_of(n, m, (int)(k / QK));
    return p.tail == 0 ? 0 : counter_bytes(p) + (size_t)p.tail * p.TS * 256 * 32 * 4;
}

template <int FMT>
static void launch_fmt(bool part, int64_t n, int nsb, const uint8_t *w, const int8_t *xq, const float *xs,
                       const _Float16 *xbs, int64_t m, float *y, int32_t *P, int32_t *M, const Plan &pl, void *ws,
                       unsigned long long seq, hipStream_t st)
{
    unsigned long long *cnt = (unsigned long long *)ws;
    float *parts = pl.tail ? (float *)((char *)ws + counter_bytes(pl)) : nullptr;
    const int64_t mtiles = (m + 255) / 256;
    const dim3 g((unsigned)(pl.full + (int64_t)pl.tail * pl.TS)), b(256);
    if (part)
        hipLaunchKernelGGL((gemm_kernel<FMT, true>), g, b, 0, st, w, n, nsb, xq, xs, xbs, m, y, P, M, (int)mtiles,
                           pl.full, pl.TS, parts, cnt, seq);
    else
        hipLaunchKernelGGL((gemm_kernel<FMT, false>), g, b, 0, st, w, n, nsb, xq, xs, xbs, m, y, P, M, (int)mtiles,
                           pl.full, pl.TS, parts, cnt, seq);
}

int launch_gemm(int fmt, const void *w, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                const void *xbs, int64_t m, float *y, int32_t *P, int32_t *M, void *ws, size_t ws_bytes,
                hipStream_t st)
{
    const int nsb = (int)(k / QK);
    const uint8_t *wb = (const uint8_t *)w;
    const _Float16 *bt = (const _Float16 *)xbs;
    const bool part = P != nullptr;
    // split only with a workspace large enough (and never for the partials)
    Plan pl = plan_of(n, m, nsb);
    if (part || !ws || ws_bytes < gemm_workspace_bytes(n, k, m) || pl.tail == 0) pl = Plan{pl.full + pl.tail, 0, 1};
    // a fresh tag per call for the split counters (48 bits used)
    static std::atomic<unsigned long long> calls{1};
    const unsigned long long seq = pl.tail ? calls.fetch_add(1, std::memory_order_relaxed) : 0;
    if (fmt == KQ_Q4_K) launch_fmt<KQ_Q4_K>(part, n, nsb, wb, xq, xs, bt, m, y, P, M, pl, ws, seq, st);
    else if (fmt == KQ_Q5_K) launch_fmt<KQ_Q5_K>(part, n, nsb, wb, xq, xs, bt, m, y, P, M, pl, ws, seq, st);
    else launch_fmt<KQ_Q6_K>(part, n, nsb, wb, xq, xs, bt, m, y, P, M, pl, ws, seq, st);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ELAUNCH;
}

}  // namespace kq
