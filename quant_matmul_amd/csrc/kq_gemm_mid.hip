// kq_gemm_mid.hip -- the K-quant x Q8_K matmul for token counts between the
// GEMV and the prefill tile (9..192 tokens), and the grouped form that runs
// every expert of a mixture-of-experts layer in one launch.
//
// Same integer partials and float fold as kq_gemm (K-quant kernel arc page,
// "The pieces", kq v2 item), the min term on v_mfma_f32_32x32x16_f16.  A
// workgroup is 4 waves over 128 weight rows x one 32-token tile (a wave: 32
// rows x 32 tokens, one v_mfma_i32_32x32x32_i8 tile), so each unpacked
// weight serves 32 tokens; what changes from the 256-token tile is how the
// weights are unpacked.  When the 32-token tiles pair up (2, 4, 5 or 6 of
// them: 33-64 and 97-192 tokens), the Q4_K/Q5_K workgroup covers 64 rows x two token tiles
// instead, so each fetched and expanded panel serves 64 tokens, and a Q6_K
// wave covers both tiles, so each digit it unpacks serves 64 tokens.
//  * Q4_K/Q5_K: a 32-weight sub-block is one K step, so the MFMA takes the
//    raw quants as its B operand, yields dot_j, and P += sc_j * dot_j is one
//    integer mad per output (cheaper at 32 tokens than folding sc_j into
//    two digit planes).  The workgroup fetches its 128 rows of a superblock
//    cooperatively (eight lanes per 128-byte row: whole cache lines) into a
//    double-buffered LDS panel of one byte per quant.
//  * Q6_K: 16-weight sub-blocks do not match a K step; each lane unpacks
//    its own half row into digit registers (kq_digits.h), no LDS panel.
// Measured on 128 experts x 32-row tiles the HBM traffic is at the
// algorithmic bytes; the per-output mads and folds keep the SIMDs, not HBM,
// the limit at this token count.
// The page's mid-size lesson (the nrsplit / regrain commits: splitting
// tokens re-ran the unpack per slice) is why a tile covers its 32 tokens in
// one pass and the grid splits rows and, when the grid is small, K -- never
// tokens.
//
// Grouped form: the activation rows are gathered per expert into one tile
// image, each expert's rows padded to whole 32-row tiles, and tile_expert
// names the expert of every 32-row tile; its weights are the planes at
// w_planes + expert * w_stride.  The page's MoE path fills one Q8_K image
// for the gate and up projections ("The pieces", kq v2 item).
#include <algorithm>
#include <type_traits>

#include "kq_common.h"
#include "kq_digits.h"

namespace kq {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

namespace {

// Q6_K raw bytes of one lane's half superblock row: lane half lh takes the
// codes k = 32*ks + 16*lh + e of every K step ks; weight 128h + 32u + 16lh
// + e is nibble u/2 of low byte 64h + 32(u%2) + 16lh + e with bits 2u, 2u+1
// of high byte 32h + 16lh + e, and its scale is that of 16-weight sub-block
// 8h + 2u + lh.
struct Lane6 {
    uint4 l[4], hq[2], sc;
    uint32_t d;
};

__device__ inline void load_lane(Lane6 &r, const uint8_t *__restrict__ w, const Planes &pl, int64_t sb, int lh)
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
__device__ inline void digits_ks(const Lane6 &r, int ks, int lh, i32x4 &bh, i32x4 &bl)
{
    uint32_t h[4], l[4];
    const int hh = ks >> 2, u = ks & 3;
    const int sc = (int8_t)byte_of(word(r.sc, (2 * ks + lh) >> 2), (2 * ks + lh) & 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lw = word(r.l[2 * hh + (u & 1)], i);
        const uint32_t nib = (u >> 1) ? (lw >> 4) & 0x0F0F0F0Fu : lw & 0x0F0F0F0Fu;
        const uint32_t q = nib | (((word(r.hq[hh], i) >> (2 * u)) & 0x03030303u) << 4);
        digits_q6(q, sc, h[i], l[i]);
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

// Q6_K form: each lane unpacks its own half superblock row straight into
// MFMA B-operand registers (no LDS panel, no barriers); its 16-weight
// sub-blocks do not match a K step, so the signed sub-scale is folded into
// two digit passes (kq_digits.h), high and low digit in two accumulators.
// With TT = 2 a wave covers two consecutive 32-token tiles, so each digit
// it unpacks feeds four MFMAs (two tiles x two digits) instead of two.
// With KP = 2 or 4 the workgroup's four waves take 4/KP row blocks of 32
// and split their K range KP ways (part p of KP*S: superblocks
// [nsb*p/(KP*S), nsb*(p+1)/(KP*S)), as the K split with KP*S parts), and
// meet in LDS, added in part order, so the workgroup writes finished sums
// (or one of S slices) instead of KP slices for the summing pass.
template <int FMT, bool GROUPED, bool PART, int TT, int KP>
__global__ __launch_bounds__(256, 2) void gemm_mid_kernel(
    const uint8_t *__restrict__ w, int64_t w_stride, const int32_t *__restrict__ tile_expert, int experts, int64_t n,
    int nsb, const int8_t *__restrict__ xq, const float *__restrict__ xs, const _Float16 *__restrict__ xbs,
    int64_t mtok, float *__restrict__ y, int32_t *__restrict__ Pout, int32_t *__restrict__ Mout, int mtiles, int S)
{
    static_assert(FMT == KQ_Q6_K, "Q4_K/Q5_K use the LDS-panel form");
    static_assert(TT == 1 || (TT == 2 && !GROUPED), "two token tiles per wave only in the plain form");
    static_assert(KP == 1 || ((KP == 2 || KP == 4) && !GROUPED && !PART), "k-parts in the plain production form only");
    constexpr int RB = 4 / KP;  // row blocks of 32 per workgroup
    __shared__ __align__(16) float d8w[4][32 * TT];
    __shared__ float red[KP > 1 ? (KP - 1) * RB : 1][TT][16][KP > 1 ? 64 : 1];  // the parts' sums

    // item = (128-row panel, 32-token tile -- or pair of tiles when TT = 2 --,
    // K split): the token tiles of a panel run on one XCD and share its L2
    // copy of the panel's planes
    const int item = item_of_mid(blockIdx.x, gridDim.x);
    const int tile = item / S, split = item - tile * S;
    // grouped: the 128-row panels of one 32-token tile (one expert) run
    // together, so they share that tile's codes and the expert's planes in
    // L2; otherwise the token tiles of one panel run together and share it
    int nt, mt;
    if constexpr (GROUPED) {
        const int ntiles = (int)((n + 127) / 128);
        mt = tile / ntiles;
        nt = tile - mt * ntiles;
    } else if constexpr (TT == 1) {
        nt = tile / mtiles;
        mt = tile - nt * mtiles;
    } else {
        const int mgroups = (mtiles + 1) / 2;
        nt = tile / mgroups;
        mt = 2 * (tile - nt * mgroups);  // the first of the wave's two token tiles
    }
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, lr = lane & 31,
              lh = lane >> 5;
    // wave wv: row block wv % RB, k-part wv / RB of this split
    const int rbk = wv % RB, kq = wv / RB;
    const int part = split * KP + kq;
    const int s0 = (int)((int64_t)nsb * part / (KP * S)), s1 = (int)((int64_t)nsb * (part + 1) / (KP * S));
    const int64_t row0 = (int64_t)nt * (32 * RB) + rbk * 32;
    // whole wave with no rows of its own (with k-parts the wave still runs,
    // clamped, to meet the workgroup's barrier)
    if (KP == 1 && row0 >= n) return;
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

    // the tile's 32 tokens of codes (tile image) and d8s; Q6_K has no min
    // term, so the bsums are not read
    (void)xbs;
    const int64_t mpad = (mtok + 31) & ~(int64_t)31;
    // token tile j of the wave: a tile past the image gets an empty range
    // (every load reads zero) based at the image start
    __amdgpu_buffer_rsrc_t rA[TT];
#pragma unroll
    for (int j = 0; j < TT; ++j) {
        const int64_t mj = m0 + 32 * j;
        const bool ok = TT == 1 || mj < mpad;
        const uint64_t a_bytes = ok ? (uint64_t)(mpad - mj) * (uint64_t)K : 0;
        rA[j] = __builtin_amdgcn_make_buffer_rsrc((void *)(xq + (ok ? mj : 0) * K), 0,
                                                  (int)(uint32_t)(a_bytes < 0xFFFFFFFFu ? a_bytes : 0xFFFFFFFFu),
                                                  0x00020000);
    }
    // token whose d8 this lane stages: lanes of half 0 for one tile, every
    // lane for two
    const int64_t td = m0 + (TT == 1 ? lr : lane);
    const float *xs_row = xs + (td < mtok ? td : mtok - 1) * nsb;

    i32x4 A[TT][8];
    Lane6 raw, nxt;
    float d8v;
    auto load_a = [&](int s, int ks) {
#pragma unroll
        for (int j = 0; j < TT; ++j)
            A[j][ks] = __builtin_bit_cast(
                i32x4, __builtin_amdgcn_raw_buffer_load_b128(rA[j], 16 * lane, (s * 8 + ks) * 1024, 0));
    };

    f32x16 accf[TT];
#pragma unroll
    for (int j = 0; j < TT; ++j) accf[j] = f32x16{};
    load_lane(raw, wb, pl, wrow + s0, lh);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) load_a(s0, ks);
    d8v = td < mtok ? xs_row[s0] : 0.0f;

    for (int s = s0; s < s1; ++s) {
        // operands of the next superblock are fetched unconditionally (the
        // last step re-reads its own, in bounds): a branch here would split
        // the K loop into blocks the scheduler cannot interleave across
        const int sn = s + 1 < s1 ? s + 1 : s;
        // stage the d8s of superblock s for the fold, 32 per token tile
        // (wave-private LDS: the wave's own later reads see these writes in
        // order)
        if (TT == 2 || lh == 0) d8w[wv][TT == 1 ? lr : lane] = d8v;
        load_lane(nxt, wb, pl, wrow + sn, lh);
        d8v = td < mtok ? xs_row[sn] : 0.0f;
        // 16-weight sub-blocks: the scale is folded into the two digit
        // passes (kq_digits.h)
        i32x16 acch[TT], accl[TT];
#pragma unroll
        for (int j = 0; j < TT; ++j) acch[j] = accl[j] = i32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            i32x4 bh, bl;
            digits_ks(raw, ks, lh, bh, bl);
#pragma unroll
            for (int j = 0; j < TT; ++j) {
                acch[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[j][ks], bh, acch[j], 0, 0, 0);
                accl[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[j][ks], bl, accl[j], 0, 0, 0);
            }
            load_a(sn, ks);
        }
        const float dv = rvalid ? f16_bits_to_float(raw.d) : 0.0f;
        __builtin_amdgcn_wave_barrier();
        // lane holds tokens 8*(i/4) + 4*lh + i%4, i = 0..15, of each tile,
        // of row `row`
#pragma unroll
        for (int j = 0; j < TT; ++j) {
            const i32x16 P = (acch[j] << 7) + accl[j];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int tl = 8 * (i >> 2) + 4 * lh + (i & 3);
                accf[j][i] = fmaf(d8w[wv][32 * j + tl], dv * (float)P[i], accf[j][i]);
                if (PART) {
                    const int64_t t = m0 + 32 * j + tl;
                    if (t < mtok && rvalid) {
                        const int64_t o = (t * n + row) * nsb + s;
                        Pout[o] = P[i];
                        if (Mout) Mout[o] = 0;
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        raw = nxt;
    }

    if constexpr (KP > 1) {
        // the parts meet: waves 1..KP-1 leave their sums in LDS, wave 0
        // adds them in part order
        if (kq > 0) {
#pragma unroll
            for (int j = 0; j < TT; ++j)
#pragma unroll
                for (int i = 0; i < 16; ++i) red[(kq - 1) * RB + rbk][j][i][lane] = accf[j][i];
        }
        __syncthreads();
        if (kq > 0) return;
#pragma unroll
        for (int q = 1; q < KP; ++q)
#pragma unroll
            for (int j = 0; j < TT; ++j)
#pragma unroll
                for (int i = 0; i < 16; ++i) accf[j][i] += red[(q - 1) * RB + rbk][j][i][lane];
    }
    // K split j of S writes slice j of y (y then points at the workspace)
    if (!rvalid) return;
    float *yo = y + (int64_t)split * mtok * n;
#pragma unroll
    for (int j = 0; j < TT; ++j) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t t = m0 + 32 * j + 8 * (i >> 2) + 4 * lh + (i & 3);
            if (t < mtok) yo[t * n + row] = accf[j][i];
        }
    }
}

// Q4_K/Q5_K form with an LDS weight panel.  The workgroup's 128 rows (64 with
// TT = 2 token tiles) x one superblock are fetched cooperatively, eight lanes per row (16 bytes each,
// so every load instruction covers eight whole 128-byte lines), expanded to
// one byte per quant into an LDS panel (row stride 272 bytes: the B-operand
// reads of 32 rows hit distinct banks) with the decoded scales, mins and
// d/dmin beside it, double-buffered with one barrier per superblock.  Each
// wave then reads its 32 rows' B operands from LDS for its token tile; the
// sub-scale is the per-output integer mad of the register form.
constexpr int MID_STRIDE = 272;

template <int FMT, bool GROUPED, bool PART, int TT>
__global__ __launch_bounds__(256, GROUPED && FMT == KQ_Q4_K ? 3 : 2) void gemm_mid_lds_kernel(
    const uint8_t *__restrict__ w, int64_t w_stride, const int32_t *__restrict__ tile_expert, int experts, int64_t n,
    int nsb, const int8_t *__restrict__ xq, const float *__restrict__ xs, const _Float16 *__restrict__ xbs,
    int64_t mtok, float *__restrict__ y, int32_t *__restrict__ Pout, int32_t *__restrict__ Mout, int mtiles, int S)
{
    static_assert(FMT != KQ_Q6_K, "Q6_K uses the register form");
    static_assert(TT == 1 || (TT == 2 && !GROUPED), "two token tiles share a panel only in the plain form");
    // TT token tiles x RW row blocks of 32 per workgroup: the panel of PR
    // rows serves 32*TT tokens
    constexpr int RW = 4 / TT, PR = 32 * RW;
    // The panel and its scales, double-buffered (one barrier per superblock)
    // -- except in the grouped Q4_K form, which keeps one buffer and takes a
    // second barrier so that three workgroups fit a CU instead of two (the
    // two staging buffers are the workgroup's whole 76 KB footprint; the
    // KHR tile page's opening change list makes the same trade).  Q5_K would
    // need more than the 168 VGPRs that three workgroups leave.
    constexpr int NB = GROUPED && FMT == KQ_Q4_K ? 1 : 2;
    __shared__ __align__(16) int8_t qp[NB][PR * MID_STRIDE];
    __shared__ __align__(16) uint32_t scw[NB][PR][2];  // 8 sub-scales per row, as bytes
    __shared__ __align__(16) uint32_t mnw[NB][PR][2];  // 8 mins per row, as bytes
    __shared__ float dd[NB][PR], dmm[NB][PR];
    __shared__ __align__(16) float d8s[NB][32 * TT];

    const int item = item_of_mid(blockIdx.x, gridDim.x);
    const int tile = item / S, split = item - tile * S;
    // grouped: the 128-row panels of one 32-token tile (one expert) run
    // together, so they share that tile's codes and the expert's planes in
    // L2; otherwise the token tiles of one panel run together and share it
    int nt, mg;
    if constexpr (GROUPED) {
        const int ntiles = (int)((n + 127) / 128);
        mg = tile / ntiles;
        nt = tile - mg * ntiles;
    } else {
        const int mgroups = (mtiles + TT - 1) / TT;
        nt = tile / mgroups;
        mg = tile - nt * mgroups;
    }
    const int s0 = (int)((int64_t)nsb * split / S), s1 = (int)((int64_t)nsb * (split + 1) / S);
    // the wave index read as uniform: the token tile, and so the tile
    // image's buffer ranges below, depend on it, and a range the compiler
    // takes for per-lane values becomes a loop over lanes at every load
    const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 31,
              lh = lane >> 5;
    // wave wv: row block wv % RW, token tile wv / RW of the group (a token
    // tile past the last one still stages and meets the barriers, its codes
    // read as zero and its outputs unstored)
    const int rb = TT == 1 ? wv : wv % RW, mt = TT == 1 ? mg : mg * TT + wv / RW;
    const int64_t n0 = (int64_t)nt * PR, m0 = (int64_t)mt * 32, mg0 = (int64_t)mg * 32 * TT;
    const uint8_t *wb = w;
    if constexpr (GROUPED) {
        const int e = tile_expert[mt];  // uniform over the workgroup
        if (e < 0 || e >= experts) return;
        wb += (int64_t)e * w_stride;
    }
    const int64_t K = (int64_t)nsb * QK;
    const Planes pl = planes_of(FMT, n, nsb);

    // panel fetch: thread covers 16 bytes (chunk tid%8) of the quant rows
    // 32j + tid/8, j < RW; threads below PR also take row tid's header
    const int chunk = tid & 7, rsub = tid >> 3;
    int64_t qrow[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) {
        const int64_t r = n0 + 32 * j + rsub;
        qrow[j] = (r < n ? r : n - 1) * nsb;
    }
    const int64_t hr = n0 + (tid & (PR - 1));
    const bool hvalid = hr < n;
    const int64_t hrow = (hvalid ? hr : n - 1) * nsb;
    uint4 rq[RW], rqh[RW], rh;
    auto fetch = [&](int s) {
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            rq[j] = *reinterpret_cast<const uint4 *>(wb + pl.off[FMT == KQ_Q5_K ? 2 : 1] + (qrow[j] + s) * 128 + 16 * chunk);
            if constexpr (FMT == KQ_Q5_K)
                rqh[j] = *reinterpret_cast<const uint4 *>(wb + pl.off[1] + (qrow[j] + s) * 32 + 16 * (chunk & 1));
        }
        rh = *reinterpret_cast<const uint4 *>(wb + pl.off[0] + (hrow + s) * 16);
    };
    // an empty asm that reads and rewrites the fetched registers: code that
    // uses them cannot be scheduled above it
    auto hold = [](uint4(&q)[RW], uint4(&qh)[RW], uint4 &h) {
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            i32x4 t = __builtin_bit_cast(i32x4, q[j]);
            asm volatile("" : "+v"(t));
            q[j] = __builtin_bit_cast(uint4, t);
            if constexpr (FMT == KQ_Q5_K) {
                i32x4 u = __builtin_bit_cast(i32x4, qh[j]);
                asm volatile("" : "+v"(u));
                qh[j] = __builtin_bit_cast(uint4, u);
            }
        }
        i32x4 t = __builtin_bit_cast(i32x4, h);
        asm volatile("" : "+v"(t));
        h = __builtin_bit_cast(uint4, t);
    };
    const int64_t td = mg0 + (tid & (32 * TT - 1));  // token whose d8 this thread stages
    const float *xs_row = xs + (td < mtok ? td : mtok - 1) * nsb;
    float d8v = 0.0f;
    // expand the fetched bytes into panel buffer b: quant byte 32c + b of a
    // row holds weight 64c + b (low nibble) and 64c + 32 + b (high nibble)
    auto stage = [&](int b) {
        const int c = chunk >> 1, b0 = 16 * (chunk & 1);
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const uint32_t q[4] = {rq[j].x, rq[j].y, rq[j].z, rq[j].w};
            uint32_t lo[4], hi[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lo[i] = q[i] & 0x0F0F0F0Fu;
                hi[i] = (q[i] >> 4) & 0x0F0F0F0Fu;
                if constexpr (FMT == KQ_Q5_K) {
                    const uint32_t hb = i == 0 ? rqh[j].x : i == 1 ? rqh[j].y : i == 2 ? rqh[j].z : rqh[j].w;
                    lo[i] |= ((hb >> (2 * c)) & 0x01010101u) << 4;
                    hi[i] |= ((hb >> (2 * c + 1)) & 0x01010101u) << 4;
                }
            }
            int8_t *row = qp[b] + (32 * j + rsub) * MID_STRIDE + 64 * c + b0;
            *reinterpret_cast<uint4 *>(row) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
            *reinterpret_cast<uint4 *>(row + 32) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        }
        if (tid < PR) {
            // rows past n: scales, mins and d masked to zero
            const uint32_t vm = hvalid ? 0xFFFFFFFFu : 0u;
            const uint32_t s0w = rh.y & vm, s1w = rh.z & vm, s2w = rh.w & vm;
            scw[b][tid][0] = s0w & 0x3F3F3F3Fu;
            scw[b][tid][1] = (s2w & 0x0F0F0F0Fu) | ((s0w >> 2) & 0x30303030u);
            mnw[b][tid][0] = s1w & 0x3F3F3F3Fu;
            mnw[b][tid][1] = ((s2w >> 4) & 0x0F0F0F0Fu) | ((s1w >> 2) & 0x30303030u);
            dd[b][tid] = f16_bits_to_float(rh.x & vm & 0xFFFFu);
            dmm[b][tid] = f16_bits_to_float((rh.x & vm) >> 16);
        }
        if (tid < 32 * TT) d8s[b][tid] = td < mtok ? d8v : 0.0f;
    };

    // the tile's 32 tokens of codes and f16 bsums (tile image)
    const int64_t mpad = (mtok + 31) & ~(int64_t)31;
    // a token tile past the image gets empty ranges (every load reads zero)
    // based at the image start
    const bool mvalid = TT == 1 || m0 < mpad;
    const int64_t mb = mvalid ? m0 : 0;
    const uint64_t a_bytes = mvalid ? (uint64_t)(mpad - m0) * (uint64_t)K : 0;
    const uint64_t b_bytes = mvalid ? (uint64_t)(mpad - m0) * (uint64_t)nsb * 32 : 0;
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xq + mb * K), 0, (int)(uint32_t)(a_bytes < 0xFFFFFFFFu ? a_bytes : 0xFFFFFFFFu), 0x00020000);
    const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xbs + mb * nsb * 16), 0, (int)(uint32_t)(b_bytes < 0xFFFFFFFFu ? b_bytes : 0xFFFFFFFFu),
        0x00020000);
    i32x4 A[8];
    f16x8 Ab;
    auto load_a = [&](int s, int ks) {
        A[ks] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, 16 * lane, (s * 8 + ks) * 1024, 0));
    };
    auto load_bs = [&](int s) {
        Ab = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(rB, 16 * lane, s * 1024, 0));
    };

    fetch(s0);
    d8v = xs_row[s0];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) load_a(s0, ks);
    load_bs(s0);
    stage(0);
    {
        const int sn = s0 + 1 < s1 ? s0 + 1 : s0;
        fetch(sn);
        d8v = xs_row[sn];
    }
    __syncthreads();

    const int rl = 32 * rb + lr;  // this lane's panel row
    const int tb = TT == 1 ? 0 : 32 * (wv / RW);  // this wave's token tile within the group's d8s
    const int64_t row = n0 + rl;
    f32x16 accf = f32x16{};
    for (int s = s0; s < s1; ++s) {
        const int b = NB == 1 ? 0 : (s - s0) & 1;
        const int sn = s + 1 < s1 ? s + 1 : s1 - 1, sn2 = s + 2 < s1 ? s + 2 : s1 - 1;
        const uint2 scv = *reinterpret_cast<const uint2 *>(scw[b][rl]);
        i32x16 P = i32x16{};
        const int8_t *brow = qp[b] + rl * MID_STRIDE + 16 * lh;
        i32x4 Bc = *reinterpret_cast<const i32x4 *>(brow);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            // the next K step's B operand is read before this step's mads
            i32x4 Bn = Bc;
            if (ks + 1 < 8) Bn = *reinterpret_cast<const i32x4 *>(brow + 32 * (ks + 1));
            const i32x16 d = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[ks], Bc, i32x16{}, 0, 0, 0);
            const int sc = (int)byte_of(ks < 4 ? scv.x : scv.y, ks & 3);
#pragma unroll
            for (int i = 0; i < 16; ++i) P[i] = __mul24(d[i], sc) + P[i];
            load_a(sn, ks);
            // keep the K steps in order (MFMA, its mads, then the next
            // step): left to itself the compiler issues all eight MFMAs
            // first and holds their 8 x 16 results live
            asm volatile("" : "+v"(P), "+v"(Bn)::"memory");
            Bc = Bn;
        }
        // min term: B operand = m of the sub-block of bsums 8lh + 0..7
        const uint32_t mw = *reinterpret_cast<const uint32_t *>(&mnw[b][rl][lh]);
        f16x8 bm;
#pragma unroll
        for (int j = 0; j < 4; ++j) bm[2 * j] = bm[2 * j + 1] = (_Float16)(int)byte_of(mw, j);
        const f32x16 mf = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ab, bm, f32x16{}, 0, 0, 0);
        load_bs(sn);
        const float dv = dd[b][rl], dm = dmm[b][rl];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int tl = 8 * (i >> 2) + 4 * lh + (i & 3);
            const float u = fmaf(dv, (float)P[i], -(dm * mf[i]));
            accf[i] = fmaf(d8s[b][tb + tl], u, accf[i]);
            if (PART) {
                const int64_t t = m0 + tl;
                if (t < mtok && row < n) {
                    const int64_t o = (t * n + row) * nsb + s;
                    Pout[o] = P[i];
                    if (Mout) Mout[o] = (int)mf[i];
                }
            }
        }
        // superblock s+1 into the other buffer (its last readers passed the
        // previous barrier; with one buffer, once every wave is done with
        // it), then fetch s+2
        if constexpr (NB == 1) __syncthreads();
        // the fetched bytes become usable only here: left to itself the
        // scheduler starts their expand among the K steps above, and the
        // wait for that fetch (issued just before the last barrier, an HBM
        // round trip) then stalls the loop's first K step
        hold(rq, rqh, rh);
        stage(NB == 1 ? 0 : b ^ 1);
        fetch(sn2);
        d8v = xs_row[sn2];
        __syncthreads();
    }

    if (row >= n) return;
    float *yo = y + (int64_t)split * mtok * n;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t t = m0 + 8 * (i >> 2) + 4 * lh + (i & 3);
        if (t < mtok) yo[t * n + row] = accf[i];
    }
}

// The paired 32-token tile (Q4_K/Q5_K, two token tiles) with its K range
// split KP ways (2 to 4) inside the workgroup: 2*KP waves, k-part q =
// wave / 2 and token tile wave % 2, each k-part with its own 32-row panel of
// its own superblock, staged together and double-buffered with one barrier
// per step.  The parts meet in LDS at the end, added in part order, so the
// workgroup writes the finished sums (or, split again across workgroups, one
// slice of them) instead of KP slices that a second pass adds.  Part p of
// KP*S covers superblocks [nsb*p/(KP*S), nsb*(p+1)/(KP*S)) as the K split of
// the 32-token tile does, so its sums are those of that split with S*KP
// parts, added in the same order.
template <int FMT, int KP>
__global__ __launch_bounds__(64 * 2 * KP, KP >= 4 ? 1 : 2) void gemm_mid_kp_kernel(
    const uint8_t *__restrict__ w, int64_t n, int nsb, const int8_t *__restrict__ xq, const float *__restrict__ xs,
    const _Float16 *__restrict__ xbs, int64_t mtok, float *__restrict__ y, int mtiles, int S)
{
    static_assert(FMT != KQ_Q6_K, "Q6_K uses the register form");
    static_assert(KP >= 2 && KP <= 4, "two to four k-parts");
    constexpr int PR = 32;
    __shared__ __align__(16) int8_t qp[2][KP][PR * MID_STRIDE];
    __shared__ __align__(16) uint32_t scw[2][KP][PR][2];
    __shared__ __align__(16) uint32_t mnw[2][KP][PR][2];
    __shared__ float dd[2][KP][PR], dmm[2][KP][PR];
    __shared__ __align__(16) float d8s[2][KP][64];

    const int item = item_of_mid(blockIdx.x, gridDim.x);
    const int tile = item / S, split = item - tile * S;
    const int mgroups = (mtiles + 1) / 2;
    const int nt = tile / mgroups, mg = tile - nt * mgroups;
    const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 31,
              lh = lane >> 5;
    const int kp = wv >> 1, tt = wv & 1;  // the wave's k-part and token tile
    const int mt = mg * 2 + tt;
    const int64_t n0 = (int64_t)nt * PR, m0 = (int64_t)mt * 32, mg0 = (int64_t)mg * 64;
    auto sbeg = [&](int q) { return (int)((int64_t)nsb * (split * KP + q) / (KP * S)); };
    int its = 0;  // steps: the longest part
#pragma unroll
    for (int q = 0; q < KP; ++q) its = max(its, sbeg(q + 1) - sbeg(q));
    const int s0 = sbeg(kp), s1 = sbeg(kp + 1);  // this wave's part
    const int64_t K = (int64_t)nsb * QK;
    const Planes pl = planes_of(FMT, n, nsb);

    // staging task: part sp = tid / 128 of the panels; 16 bytes (chunk u%8)
    // of rows u/8 and u/8 + 16 of that part's panel; u < 32 also takes row
    // u's header, u < 64 the d8 of the group's token u
    const int sp = tid >> 7, u = tid & 127, chunk = u & 7, rsub = u >> 3;
    const int ps0 = sbeg(sp), ps1 = sbeg(sp + 1);
    auto sb_of = [&](int it) { return min(ps0 + it, ps1 - 1); };  // staged superblock of step it, clamped
    int64_t qrow[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t r = n0 + 16 * j + rsub;
        qrow[j] = (r < n ? r : n - 1) * nsb;
    }
    const int64_t hr = n0 + (u & (PR - 1));
    const bool hvalid = hr < n;
    const int64_t hrow = (hvalid ? hr : n - 1) * nsb;
    const int64_t td = mg0 + (u & 63);  // token whose d8 this thread stages
    const float *xs_row = xs + (td < mtok ? td : mtok - 1) * nsb;
    uint4 rq[2], rqh[2], rh;
    float d8v;
    auto fetch = [&](int it) {
        const int s = sb_of(it);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            rq[j] = *reinterpret_cast<const uint4 *>(w + pl.off[FMT == KQ_Q5_K ? 2 : 1] + (qrow[j] + s) * 128 + 16 * chunk);
            if constexpr (FMT == KQ_Q5_K)
                rqh[j] = *reinterpret_cast<const uint4 *>(w + pl.off[1] + (qrow[j] + s) * 32 + 16 * (chunk & 1));
        }
        rh = *reinterpret_cast<const uint4 *>(w + pl.off[0] + (hrow + s) * 16);
        d8v = xs_row[s];
    };
    // the fetched registers pass an empty asm before the expand, so it is
    // not scheduled among the K steps (where the wait for the fetch would
    // stall them)
    auto hold = [&]() {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            i32x4 t = __builtin_bit_cast(i32x4, rq[j]);
            asm volatile("" : "+v"(t));
            rq[j] = __builtin_bit_cast(uint4, t);
            if constexpr (FMT == KQ_Q5_K) {
                i32x4 v = __builtin_bit_cast(i32x4, rqh[j]);
                asm volatile("" : "+v"(v));
                rqh[j] = __builtin_bit_cast(uint4, v);
            }
        }
        i32x4 t = __builtin_bit_cast(i32x4, rh);
        asm volatile("" : "+v"(t), "+v"(d8v));
        rh = __builtin_bit_cast(uint4, t);
    };
    // expand into buffer b of part sp's panel: quant byte 32c + b of a row
    // holds weight 64c + b (low nibble) and 64c + 32 + b (high nibble)
    auto stage = [&](int b) {
        const int c = chunk >> 1, b0 = 16 * (chunk & 1);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t q[4] = {rq[j].x, rq[j].y, rq[j].z, rq[j].w};
            uint32_t lo[4], hi[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lo[i] = q[i] & 0x0F0F0F0Fu;
                hi[i] = (q[i] >> 4) & 0x0F0F0F0Fu;
                if constexpr (FMT == KQ_Q5_K) {
                    const uint32_t hb = i == 0 ? rqh[j].x : i == 1 ? rqh[j].y : i == 2 ? rqh[j].z : rqh[j].w;
                    lo[i] |= ((hb >> (2 * c)) & 0x01010101u) << 4;
                    hi[i] |= ((hb >> (2 * c + 1)) & 0x01010101u) << 4;
                }
            }
            int8_t *row = qp[b][sp] + (16 * j + rsub) * MID_STRIDE + 64 * c + b0;
            *reinterpret_cast<uint4 *>(row) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
            *reinterpret_cast<uint4 *>(row + 32) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        }
        if (u < PR) {
            // rows past n: scales, mins and d masked to zero
            const uint32_t vm = hvalid ? 0xFFFFFFFFu : 0u;
            const uint32_t s0w = rh.y & vm, s1w = rh.z & vm, s2w = rh.w & vm;
            scw[b][sp][u][0] = s0w & 0x3F3F3F3Fu;
            scw[b][sp][u][1] = (s2w & 0x0F0F0F0Fu) | ((s0w >> 2) & 0x30303030u);
            mnw[b][sp][u][0] = s1w & 0x3F3F3F3Fu;
            mnw[b][sp][u][1] = ((s2w >> 4) & 0x0F0F0F0Fu) | ((s1w >> 2) & 0x30303030u);
            dd[b][sp][u] = f16_bits_to_float(rh.x & vm & 0xFFFFu);
            dmm[b][sp][u] = f16_bits_to_float((rh.x & vm) >> 16);
        }
        if (u < 64) d8s[b][sp][u] = td < mtok ? d8v : 0.0f;
    };

    // the wave's token tile of codes and f16 bsums (a tile past the image
    // gets empty ranges: every load reads zero)
    const int64_t mpad = (mtok + 31) & ~(int64_t)31;
    const bool mvalid = m0 < mpad;
    const int64_t mb = mvalid ? m0 : 0;
    const uint64_t a_bytes = mvalid ? (uint64_t)(mpad - m0) * (uint64_t)K : 0;
    const uint64_t b_bytes = mvalid ? (uint64_t)(mpad - m0) * (uint64_t)nsb * 32 : 0;
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xq + mb * K), 0, (int)(uint32_t)(a_bytes < 0xFFFFFFFFu ? a_bytes : 0xFFFFFFFFu), 0x00020000);
    const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(xbs + mb * nsb * 16), 0, (int)(uint32_t)(b_bytes < 0xFFFFFFFFu ? b_bytes : 0xFFFFFFFFu),
        0x00020000);
    i32x4 A[8];
    f16x8 Ab;
    auto load_a = [&](int s, int ks) {
        A[ks] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, 16 * lane, (s * 8 + ks) * 1024, 0));
    };
    auto load_bs = [&](int s) {
        Ab = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(rB, 16 * lane, s * 1024, 0));
    };

    fetch(0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) load_a(s0, ks);
    load_bs(s0);
    stage(0);
    fetch(1);
    __syncthreads();

    const int rl = lr;  // this lane's panel row
    const int64_t row = n0 + rl;
    f32x16 accf = f32x16{};
    for (int it = 0; it < its; ++it) {
        const int b = it & 1;
        const bool live = s0 + it < s1;  // a shorter part idles on the longest part's last step
        const int sw = min(s0 + it + 1, s1 - 1);  // the next step's codes (clamped)
        const uint2 scv = *reinterpret_cast<const uint2 *>(scw[b][kp][rl]);
        i32x16 P = i32x16{};
        const int8_t *brow = qp[b][kp] + rl * MID_STRIDE + 16 * lh;
        i32x4 Bc = *reinterpret_cast<const i32x4 *>(brow);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            i32x4 Bn = Bc;
            if (ks + 1 < 8) Bn = *reinterpret_cast<const i32x4 *>(brow + 32 * (ks + 1));
            const i32x16 d = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[ks], Bc, i32x16{}, 0, 0, 0);
            const int sc = (int)byte_of(ks < 4 ? scv.x : scv.y, ks & 3);
#pragma unroll
            for (int i = 0; i < 16; ++i) P[i] = __mul24(d[i], sc) + P[i];
            load_a(sw, ks);
            asm volatile("" : "+v"(P), "+v"(Bn)::"memory");
            Bc = Bn;
        }
        const uint32_t mw = *reinterpret_cast<const uint32_t *>(&mnw[b][kp][rl][lh]);
        f16x8 bm;
#pragma unroll
        for (int j = 0; j < 4; ++j) bm[2 * j] = bm[2 * j + 1] = (_Float16)(int)byte_of(mw, j);
        const f32x16 mf = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ab, bm, f32x16{}, 0, 0, 0);
        load_bs(sw);
        const float dv = dd[b][kp][rl], dm = dmm[b][kp][rl];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int tl = 8 * (i >> 2) + 4 * lh + (i & 3);
            const float uu = fmaf(dv, (float)P[i], -(dm * mf[i]));
            const float a = fmaf(d8s[b][kp][32 * tt + tl], uu, accf[i]);
            accf[i] = live ? a : accf[i];
        }
        // step it+1 into the other buffers (their last readers passed the
        // previous barrier), then fetch step it+2
        hold();
        stage(b ^ 1);
        fetch(it + 2);
        __syncthreads();
    }

    // the parts meet: parts 1..KP-1 leave their sums in LDS (the panel
    // buffers, free after the last barrier), part 0 adds them in order
    static_assert(sizeof(qp) >= sizeof(float) * (KP - 1) * 2 * 16 * 64, "the parts' sums fit the panel buffers");
    float *red = reinterpret_cast<float *>(&qp[0][0][0]);
    if (kp > 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) red[(((kp - 1) * 2 + tt) * 16 + i) * 64 + lane] = accf[i];
    }
    __syncthreads();
    if (kp > 0 || row >= n) return;
#pragma unroll
    for (int q = 1; q < KP; ++q)
#pragma unroll
        for (int i = 0; i < 16; ++i) accf[i] += red[(((q - 1) * 2 + tt) * 16 + i) * 64 + lane];
    float *yo = y + (int64_t)split * mtok * n;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t t = m0 + 8 * (i >> 2) + 4 * lh + (i & 3);
        if (t < mtok) yo[t * n + row] = accf[i];
    }
}

void launch_sum_splits(const float *p, int S, int64_t count, float *y, hipStream_t st);
int cu_count();

namespace {

int pick_splits_mid(int64_t waves, int nsb)
{
    const int cus = cu_count();
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
    const int64_t mtiles = (m + 31) / 32;
    // token tiles pair up, on 64-row panels (Q4_K/Q5_K) or within each wave
    // (Q6_K), when their count is even or five (129-160 tokens: three pairs,
    // the last one's second tile empty, beat five single tiles -- except for
    // Q6_K split along k, whose half-empty last pair costs more than it saves)
    // The Q6_K partials (a test path) run unpaired: the paired register
    // form with the partials stores spills.  Each output's fold runs over
    // the same superblocks in the same order either way, so y is the same.
    const bool pair = !GROUPED && (mtiles % 2 == 0 || (mtiles == 5 && (FMT != KQ_Q6_K || S == 1))) &&
                      !(FMT == KQ_Q6_K && part);
    const int64_t ntiles = pair && FMT != KQ_Q6_K ? (n + 63) / 64 : (n + 127) / 128;
    const dim3 g((unsigned)(ntiles * (pair ? (mtiles + 1) / 2 : mtiles) * S)), b(256);
    if constexpr (FMT == KQ_Q6_K) {
        if constexpr (!GROUPED) {
            if (pair) {
                hipLaunchKernelGGL((gemm_mid_kernel<FMT, false, false, 2, 1>), g, b, 0, st, w, w_stride, tile_expert,
                                   experts, n, nsb, xq, xs, xbs, m, y, P, M, (int)mtiles, S);
                return;
            }
        }
        if (part)
            hipLaunchKernelGGL((gemm_mid_kernel<FMT, GROUPED, !GROUPED, 1, 1>), g, b, 0, st, w, w_stride, tile_expert, experts,
                               n, nsb, xq, xs, xbs, m, y, P, M, (int)mtiles, S);
        else
            hipLaunchKernelGGL((gemm_mid_kernel<FMT, GROUPED, false, 1, 1>), g, b, 0, st, w, w_stride, tile_expert,
                               experts, n, nsb, xq, xs, xbs, m, y, P, M, (int)mtiles, S);
    } else {
        if constexpr (!GROUPED) {
            if (pair) {
                if (part)
                    hipLaunchKernelGGL((gemm_mid_lds_kernel<FMT, false, true, 2>), g, b, 0, st, w, w_stride,
                                       tile_expert, experts, n, nsb, xq, xs, xbs, m, y, P, M, (int)mtiles, S);
                else
                    hipLaunchKernelGGL((gemm_mid_lds_kernel<FMT, false, false, 2>), g, b, 0, st, w, w_stride,
                                       tile_expert, experts, n, nsb, xq, xs, xbs, m, y, P, M, (int)mtiles, S);
                return;
            }
        }
        if (part)
            hipLaunchKernelGGL((gemm_mid_lds_kernel<FMT, GROUPED, !GROUPED, 1>), g, b, 0, st, w, w_stride, tile_expert,
                               experts, n, nsb, xq, xs, xbs, m, y, P, M, (int)mtiles, S);
        else
            hipLaunchKernelGGL((gemm_mid_lds_kernel<FMT, GROUPED, false, 1>), g, b, 0, st, w, w_stride, tile_expert,
                               experts, n, nsb, xq, xs, xbs, m, y, P, M, (int)mtiles, S);
    }
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

// four-wave k-part workgroups (KP = 2) held per CU in one round: their
// 149-161 VGPRs leave room for three waves per SIMD
constexpr int KP_PER_CU = 3;

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
    // a NULL or too small workspace runs the tile unsplit (bitwise the
    // partials kernel's outputs)
    const bool split_ok = !part && ws && ws_bytes >= gemm_mid_workspace_bytes(n, k, m);
    const int S = split_ok ? pick_splits_mid(mid_waves(n, m), nsb) : 1;
    // A Q4_K/Q5_K paired tile split along k runs KP of its parts inside each
    // workgroup (gemm_mid_kp_kernel) and Sw slices across workgroups, so the
    // summing pass adds fewer slices, or none -- while its grid runs in one
    // round.  KP = 4 (eight waves, one workgroup per CU) takes as many
    // slices as fill the CUs once, where that is at least two (W_down at up
    // to 64 tokens: 240 workgroups of three slices), or one where the tiles
    // alone take three quarters of the CUs.  KP = 3 takes S/3
    // (rounded) slices, at most one six-wave workgroup per CU (at 320
    // workgroups, W_down at 100-160 tokens, the CUs given two set the end:
    // 22.4 -> 32.4 us).  KP = 2 takes S/2 slices, KP_PER_CU four-wave
    // workgroups per CU; an unsplit tile (S = 1) runs as two parts where
    // that grid fits (W_up at 100-128 tokens: 20.8 -> 18.8 us on Q4_K).  An
    // odd tile count pairs its last tile with an empty one (codes read as
    // zero, outputs unstored): three tiles (65-96 tokens) take the pairs
    // (W_up 21.5 -> 17.6 us on Q4_K), one tile (up to 32 tokens) only with
    // four parts (W_down 15.4 -> 14.6 us; two parts and two slices were
    // slower on W_up).
    const int64_t mtiles = (m + 31) / 32;
    if (split_ok && fmt != KQ_Q6_K) {
        const int64_t cells = ((n + 31) / 32) * ((mtiles + 1) / 2);
        for (int kp = 4; kp >= 2; --kp) {
            if (mtiles == 1 && kp != 4) continue;
            int Sw;
            if (kp == 4) {
                if (S < 4) continue;
                Sw = (int)std::min<int64_t>(cu_count() / cells, S);
            } else {
                if (S < kp && !(S == 1 && kp == 2)) continue;
                Sw = (S + (kp == 3 ? 1 : 0)) / kp;  // three parts: rounded; two: floor, so S = 3 stays in one slice
                Sw = Sw > 1 ? Sw : 1;
            }
            while (Sw > 1 && kp * Sw > nsb) --Sw;
            // one slice only where the cells alone nearly fill the CUs (W_down at
            // 129-192 tokens, 240 cells: 27.3 -> 22.8 us on Q4_K at 160 tokens;
            // at 160 cells, 100-128 tokens, two parts and three slices stay faster)
            if (kp == 4 && Sw < 2 && !(Sw == 1 && 4 * cells >= 3 * (int64_t)cu_count())) continue;
            const int64_t grid = cells * Sw;
            if (kp * Sw > nsb || grid > (kp == 2 ? KP_PER_CU : 1) * (int64_t)cu_count()) continue;
            float *dst = Sw > 1 ? (float *)ws : y;
            const dim3 g((unsigned)grid), b(64 * 2 * kp);
            auto go = [&](auto f, auto k) {
                hipLaunchKernelGGL((gemm_mid_kp_kernel<decltype(f)::value, decltype(k)::value>), g, b, 0, st,
                                   (const uint8_t *)w, n, nsb, xq, xs, (const _Float16 *)xbs, m, dst, (int)mtiles, Sw);
            };
            using I4 = std::integral_constant<int, KQ_Q4_K>;
            using I5 = std::integral_constant<int, KQ_Q5_K>;
            using K2 = std::integral_constant<int, 2>;
            using K3 = std::integral_constant<int, 3>;
            using K4 = std::integral_constant<int, 4>;
            if (fmt == KQ_Q4_K) kp == 4 ? go(I4{}, K4{}) : kp == 3 ? go(I4{}, K3{}) : go(I4{}, K2{});
            else kp == 4 ? go(I5{}, K4{}) : kp == 3 ? go(I5{}, K3{}) : go(I5{}, K2{});
            if (Sw > 1) launch_sum_splits((const float *)ws, Sw, m * n, y, st);
            return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ELAUNCH;
        }
    }
    // Q6_K split along k: the register tile's four waves take 4/KP row
    // blocks and KP of the parts (gemm_mid_kernel, KP = 4, else 2), S/KP
    // (or, for KP = 4, enough to fill the CUs) across workgroups, while the grid holds at most one workgroup per CU
    // (its 241 VGPRs leave room for two waves per SIMD, but with more
    // workgroups than CUs the CUs given two set the end: W_down at 100-128
    // tokens, 25.4 -> 29.9 us)
    if (split_ok && fmt == KQ_Q6_K && S >= 2) {
        // token tiles paired as launch_mid_fmt pairs a split Q6_K tile, and
        // five tiles too, the last pair's second tile empty (W_down at 129-160
        // tokens: four parts on 240 workgroups, 35.3 -> 26.3 us)
        const bool pair6 = mtiles % 2 == 0 || mtiles == 5;
        for (int kp = 4; kp >= 2; kp -= 2) {
            if (S < kp) continue;
            int S6 = (S + (kp == 4 ? 2 : 0)) / kp;  // four parts: rounded; two: floor
            S6 = S6 > 1 ? S6 : 1;
            if (kp == 4) {  // or as many slices as fill the CUs once, if more (W_down at up to 64 tokens: three)
                const int64_t cells = ((n + 31) / 32) * (pair6 ? (mtiles + 1) / 2 : mtiles);
                const int sf = (int)(cu_count() / cells);
                if (sf > S6 && sf <= S) S6 = sf;
            }
            while (S6 > 1 && kp * S6 > nsb) --S6;
            const int64_t grid = ((n + 32 * (4 / kp) - 1) / (32 * (4 / kp))) * (pair6 ? (mtiles + 1) / 2 : mtiles) * S6;
            if (kp * S6 > nsb || grid > cu_count()) continue;
            float *dst = S6 > 1 ? (float *)ws : y;
            const dim3 g((unsigned)grid), b(256);
            auto go = [&](auto tt, auto k) {
                hipLaunchKernelGGL((gemm_mid_kernel<KQ_Q6_K, false, false, decltype(tt)::value, decltype(k)::value>), g,
                                   b, 0, st, (const uint8_t *)w, 0, nullptr, 0, n, nsb, xq, xs, (const _Float16 *)xbs, m,
                                   dst, nullptr, nullptr, (int)mtiles, S6);
            };
            using T1 = std::integral_constant<int, 1>;
            using T2 = std::integral_constant<int, 2>;
            using K4 = std::integral_constant<int, 4>;
            if (pair6) kp == 4 ? go(T2{}, K4{}) : go(T2{}, T2{});
            else kp == 4 ? go(T1{}, K4{}) : go(T1{}, T2{});
            if (S6 > 1) launch_sum_splits((const float *)ws, S6, m * n, y, st);
            return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ELAUNCH;
        }
    }
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
