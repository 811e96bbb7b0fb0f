// kq_gemv_mma.hip -- decode GEMV for batches 3-8 on the matrix cores (gfx950).
//
// The same sums as kq_gemv.hip (K-quant kernel arc page, "The pieces", kq v2
// item; k4 v2 and k5/k6 v2 commit messages): per (token, row, superblock)
// the sub-scale x int32 dot and the min x bsum terms in integers, then ONE
// float fold.  Past two tokens the sdot4 GEMV's per-token work (16 dot4 per
// lane and 64 weights, plus the codes re-read from LDS by every row of a
// quad group) grows with the batch while the weight bytes do not; here the
// contraction over a sub-block runs on v_mfma_i32_16x16x32_i8 instead:
//
//   D[t][r] = sum over the 32 weights of sub-block j of a_t[i] * q_r[i]
//
// for 16 token slots t (A operand: the Q8_K codes) and 16 rows r (B operand:
// the raw 4/5/6-bit quants), and the lane that holds row r's quants also
// holds D[4g .. 4g+3][r] (g = lane / 16), so the row's scales, decoded in
// that lane, apply in the epilogue:
//
//   Q4_K / Q5_K:  P = sum_j sc_j * D_j (24-bit integer mads: |D_j| < 2^17),
//                 M = sum_g m_{g/2} * bsum_g  on v_mfma_f32_16x16x16_f16
//                     (exact: |bsum| <= 2032 and m <= 63 are f16 integers,
//                     |M| < 2^24);
//   Q6_K:         16-wide sub-blocks.  At most 8 tokens fill half the 16
//                 token slots, so slot i < 8 carries token i over a chunk's
//                 first 16 weights and slot 8 + i the same token over the
//                 last 16 (the rest of each A row zero): one MFMA per chunk
//                 gives both sub-blocks' dots.  P = sum_b sc_b * D_b - 32 * B,
//                 B = sum_b sc_b * bsum_b on the f16 matrix core (|B| < 2^23).
//
// Operand layouts (checked on the device): 16x16x32 i8 -- A[i][k]: lane l
// holds i = l % 16, k = 8*(l/16) .. +7; B[k][j]: j = l % 16, the same k;
// D[i][j]: j = l % 16, i = 4*(l/16) .. +3.  16x16x16 f16 -- the same with
// k = 4*(l/16) .. +3.
//
// Work: a wave covers 16 rows and a contiguous run of superblocks; the kw
// waves of a workgroup split the row group's superblocks and meet in LDS in
// wave order.  Codes, bsums and scales come from the Q8_K row image in L2
// (every wave reads the codes of its superblocks once); each wave stages
// one superblock's weights and codes in its own LDS area and keeps the
// next superblock's loads in flight while it folds the current one.
#include <type_traits>

#include "kq_common.h"

namespace kq {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

__device__ inline v4i mma_i8(uint2 a, uint2 b)
{
    long av, bv;
    __builtin_memcpy(&av, &a, 8);
    __builtin_memcpy(&bv, &b, 8);
    const v4i z = {0, 0, 0, 0};
    return __builtin_amdgcn_mfma_i32_16x16x32_i8(av, bv, z, 0, 0, 0);
}

__device__ inline v4f mma_f16(v4h a, v4h b)
{
    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, z, 0, 0, 0);
}

// Each wave stages what it needs for one superblock in its own LDS area:
// the global loads are laid out for coalescing (consecutive lanes read
// consecutive bytes of a row), while the matrix-core operands want lane
// l to hold row (or token) l % 16 -- sixteen different rows per 16 lanes,
// which read straight from global memory would not coalesce at all.
// Row strides are padded so that the operand reads (16 lanes, 16 rows, 8
// bytes each) hit distinct banks.
constexpr int QS = 136;   // a row's 128 quant bytes (Q4_K/Q5_K qs, Q6_K ql)
constexpr int QHS = 72;   // a Q6_K row's 64 high-bit bytes
constexpr int Q5S = 40;   // a Q5_K row's 32 fifth-bit bytes
constexpr int CS = 264;   // a token's 256 codes
constexpr int TMAX = 8;   // token slots staged (the batch)

template <int FMT>
struct Lay;  // byte offsets of the parts of a wave's LDS area
template <>
struct Lay<KQ_Q4_K> {
    static constexpr int q = 0, h = 16 * QS, c = h + 256, b = c + TMAX * CS, d = b + TMAX * 32, size = d + 64;
};
template <>
struct Lay<KQ_Q5_K> {
    static constexpr int q = 0, qh = 16 * QS, h = qh + 16 * Q5S, c = h + 256, b = c + TMAX * CS, d = b + TMAX * 32,
                         size = d + 64;
};
template <>
struct Lay<KQ_Q6_K> {
    static constexpr int q = 0, qh = 16 * QS, h = qh + 16 * QHS, dd = h + 256, c = dd + 64, b = c + TMAX * CS,
                         d = b + TMAX * 32, size = d + 64;
};

// The global loads of one superblock, held in registers until staged:
// lane l takes row l / 4, bytes 32 (l % 4) .. +31 of its quant bytes; the
// small fields (scales, fifth or high bits, codes, bsums, d8) by the lanes
// that own them.
template <int FMT>
struct Fetch {
    uint4 q0, q1;   // quant bytes
    uint4 x;        // Q5_K fifth bits / Q6_K high bits (lane l: row l / 2 or l / 4)
    uint4 h;        // row l % 16's 16 header (or Q6_K scale) bytes
    uint32_t dd;    // Q6_K: row l % 16's f16 d
    uint4 c0, c1;   // codes: lane l, token l / 16 (+ 4), bytes 16 (l % 16) .. +15
    uint4 b;        // token (l / 2) % 8, bsums 8 (l % 2) .. +7
    float d8;       // token l % 8's scale
};

template <int FMT>
__device__ inline void fetch(Fetch<FMT> &r, const uint8_t *__restrict__ w, const Planes &pl, int64_t rowsb0,
                                int nsb, int64_t rows_left, int s, const int8_t *__restrict__ xq,
                                const float *__restrict__ xs, const int16_t *__restrict__ xbs, int T, int lane)
{
    // row l / 4 of the group (rows past n re-read the group's first row)
    const int rl = lane >> 2;
    const int64_t sb = rowsb0 + (int64_t)(rl < rows_left ? rl : 0) * nsb + s;
    const uint8_t *q = w + pl.off[FMT == KQ_Q6_K ? 0 : (FMT == KQ_Q5_K ? 2 : 1)] + sb * 128 + 32 * (lane & 3);
    r.q0 = *reinterpret_cast<const uint4 *>(q);
    r.q1 = *reinterpret_cast<const uint4 *>(q + 16);
    if constexpr (FMT == KQ_Q5_K) {
        // lanes 0..31: row l / 2, fifth-bit bytes 16 (l % 2) .. +15
        const int r2 = (lane >> 1) & 15;
        const int64_t s2 = rowsb0 + (int64_t)(r2 < rows_left ? r2 : 0) * nsb + s;
        r.x = *reinterpret_cast<const uint4 *>(w + pl.off[1] + s2 * 32 + 16 * (lane & 1));
    }
    if constexpr (FMT == KQ_Q6_K) {
        // row l / 4, high-bit bytes 16 (l % 4) .. +15
        r.x = *reinterpret_cast<const uint4 *>(w + pl.off[1] + sb * 64 + 16 * (lane & 3));
    }
    const int r16 = lane & 15;
    const int64_t s16 = rowsb0 + (int64_t)(r16 < rows_left ? r16 : 0) * nsb + s;
    r.h = *reinterpret_cast<const uint4 *>(w + pl.off[FMT == KQ_Q6_K ? 2 : 0] + s16 * 16);
    if constexpr (FMT == KQ_Q6_K) r.dd = *reinterpret_cast<const uint16_t *>(w + pl.off[3] + s16 * 2);
    // codes of tokens l / 16 and 4 + l / 16 (past the batch: the last token)
    const int64_t K = (int64_t)nsb * QK;
    const int t0 = min(lane >> 4, T - 1), t1 = min(4 + (lane >> 4), T - 1);
    r.c0 = *reinterpret_cast<const uint4 *>(xq + t0 * K + (int64_t)s * QK + 16 * (lane & 15));
    r.c1 = *reinterpret_cast<const uint4 *>(xq + t1 * K + (int64_t)s * QK + 16 * (lane & 15));
    const int tb = min((lane >> 1) & 7, T - 1);
    r.b = *reinterpret_cast<const uint4 *>(xbs + tb * (K / 16) + (int64_t)s * 16 + 8 * (lane & 1));
    r.d8 = xs[(int64_t)min(lane & 7, T - 1) * nsb + s];
}

template <int FMT>
__device__ inline void stage_lds(const Fetch<FMT> &r, uint8_t *__restrict__ L, int lane)
{
    using Y = Lay<FMT>;
    const int rl = lane >> 2;
    uint2 *q = reinterpret_cast<uint2 *>(L + Y::q + rl * QS + 32 * (lane & 3));
    q[0] = make_uint2(r.q0.x, r.q0.y);
    q[1] = make_uint2(r.q0.z, r.q0.w);
    q[2] = make_uint2(r.q1.x, r.q1.y);
    q[3] = make_uint2(r.q1.z, r.q1.w);
    if constexpr (FMT == KQ_Q5_K) {
        uint2 *x = reinterpret_cast<uint2 *>(L + Y::qh + ((lane >> 1) & 15) * Q5S + 16 * (lane & 1));
        x[0] = make_uint2(r.x.x, r.x.y);
        x[1] = make_uint2(r.x.z, r.x.w);
    }
    if constexpr (FMT == KQ_Q6_K) {
        uint2 *x = reinterpret_cast<uint2 *>(L + Y::qh + rl * QHS + 16 * (lane & 3));
        x[0] = make_uint2(r.x.x, r.x.y);
        x[1] = make_uint2(r.x.z, r.x.w);
        reinterpret_cast<uint32_t *>(L + Y::dd)[lane & 15] = r.dd;
    }
    // the small fields: every lane stores (lanes 16 apart hold the same
    // bytes), so no store is conditional
    reinterpret_cast<uint4 *>(L + Y::h)[lane & 15] = make_uint4(r.h.x, r.h.y, r.h.z, r.h.w);
    uint2 *c0 = reinterpret_cast<uint2 *>(L + Y::c + (lane >> 4) * CS + 16 * (lane & 15));
    c0[0] = make_uint2(r.c0.x, r.c0.y);
    c0[1] = make_uint2(r.c0.z, r.c0.w);
    uint2 *c1 = reinterpret_cast<uint2 *>(L + Y::c + (4 + (lane >> 4)) * CS + 16 * (lane & 15));
    c1[0] = make_uint2(r.c1.x, r.c1.y);
    c1[1] = make_uint2(r.c1.z, r.c1.w);
    reinterpret_cast<uint4 *>(L + Y::b)[lane & 15] = make_uint4(r.b.x, r.b.y, r.b.z, r.b.w);
    reinterpret_cast<float *>(L + Y::d)[lane & 7] = r.d8;
}

__device__ inline v4h bsums_f16(uint2 b)
{
    v4h v;
    v[0] = (_Float16)(int16_t)(b.x & 0xFFFF);
    v[1] = (_Float16)(int16_t)(b.x >> 16);
    v[2] = (_Float16)(int16_t)(b.y & 0xFFFF);
    v[3] = (_Float16)(int16_t)(b.y >> 16);
    return v;
}

__device__ inline uint2 lds8(const uint8_t *p) { return *reinterpret_cast<const uint2 *>(p); }

// P[i] and the float M[i] (exact integer) of tokens 4g + i for row r16 of
// the group from the staged superblock; d, dmin the row's scales.  ta is
// the lane's A-operand token slot (past the batch: the last token).
template <int FMT>
__device__ inline void superblock(const uint8_t *__restrict__ L, int r16, int g, int ta, int (&P)[4], float (&M)[4],
                                  float &d, float &dmin)
{
    using Y = Lay<FMT>;
#pragma unroll
    for (int i = 0; i < 4; ++i) P[i] = 0;
    const uint8_t *cb = L + Y::c + ta * CS + 8 * g;  // codes: + 32 j
    const v4h ab = bsums_f16(lds8(L + Y::b + ta * 32 + 8 * g));
    const uint8_t *qb = L + Y::q + r16 * QS + 8 * g;
    if constexpr (FMT == KQ_Q6_K) {
        // A chunk of 32 weights holds two 16-wide sub-blocks, each with its
        // own scale.  The token slots carry both: slot i < 8 is token i over
        // the chunk's first 16 k-slots (the other 16 zero), slot 8 + i the
        // same token over the last 16, so one MFMA gives D[i][r] = the dot
        // of sub-block 2c and D[8 + i][r] that of 2c + 1.  Lane (r, g) then
        // holds tokens 4 (g & 1) .. +3 of sub-block 2c + (g >> 1): one scale
        // per lane, and the two halves of a token's P sit in lanes g and g ^ 2.
        d = f16_bits_to_float(reinterpret_cast<const uint32_t *>(L + Y::dd)[r16] & 0xFFFFu);
        dmin = 0.0f;
        const uint4 sc = reinterpret_cast<const uint4 *>(L + Y::h)[r16];
        const uint32_t scw[4] = {sc.x, sc.y, sc.z, sc.w};
        const uint2 hb0 = lds8(L + Y::qh + r16 * QHS + 8 * g), hb1 = lds8(L + Y::qh + r16 * QHS + 32 + 8 * g);
        const uint32_t amask = ((g < 2) == (r16 < 8)) ? 0xFFFFFFFFu : 0u;
        const uint8_t *c6 = L + Y::c + ta * CS + 8 * g;
        const int half = g >> 1;
        // chunk c = 4h + cc: low (cc < 2) or high nibbles of ql bytes
        // 64h + 32 (cc & 1) + ..., high bits 2cc .. 2cc+1 of qh bytes 32h + ...
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int h = c >> 2, cc = c & 3;
            const uint2 l = lds8(qb + 64 * h + 32 * (cc & 1));
            const uint32_t n0 = (cc >> 1) ? (l.x >> 4) & 0x0F0F0F0Fu : l.x & 0x0F0F0F0Fu;
            const uint32_t n1 = (cc >> 1) ? (l.y >> 4) & 0x0F0F0F0Fu : l.y & 0x0F0F0F0Fu;
            const uint2 hb = h ? hb1 : hb0;
            const uint32_t q0 = n0 | (((hb.x >> (2 * cc)) & 0x03030303u) << 4);
            const uint32_t q1 = n1 | (((hb.y >> (2 * cc)) & 0x03030303u) << 4);
            const uint2 a = lds8(c6 + 32 * c);
            const v4i D = mma_i8(make_uint2(a.x & amask, a.y & amask), make_uint2(q0, q1));
            const uint32_t sw = scw[c >> 1];
            const int sl = (int8_t)byte_of(sw, 2 * (c & 1)), sh = (int8_t)byte_of(sw, 2 * (c & 1) + 1);
            const int sb = half ? sh : sl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                P[i] += __mul24(sb, D[i]);
                // one chunk's operands live at a time (hoisting all eight
                // chunks' LDS reads costs occupancy)
                asm volatile("" : "+v"(P[i]));
            }
        }
        // B = sum_b sc_b * bsum_b on the f16 core (lane k-slots 4g .. 4g+3 are
        // sub-blocks 4g .. 4g+3), subtracted once per token: in the half g < 2
        const uint32_t sg = g == 0 ? sc.x : g == 1 ? sc.y : g == 2 ? sc.z : sc.w;
        v4h bs;
#pragma unroll
        for (int e = 0; e < 4; ++e) bs[e] = (_Float16)(int8_t)byte_of(sg, e);
        const v4f B = mma_f16(ab, bs);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (half == 0) P[i] -= 32 * (int)B[i];
            M[i] = 0.0f;
        }
    } else {
        const uint4 h = reinterpret_cast<const uint4 *>(L + Y::h)[r16];
        d = f16_bits_to_float(h.x & 0xFFFFu);
        dmin = f16_bits_to_float(h.x >> 16);
        // the 6-bit packing, four sub-blocks per dword (byte j of each)
        const uint32_t s0 = h.y, s1 = h.z, s2 = h.w;
        const uint32_t scA = s0 & 0x3F3F3F3Fu, mA = s1 & 0x3F3F3F3Fu;
        const uint32_t scB = (s2 & 0x0F0F0F0Fu) | ((s0 >> 2) & 0x30303030u);
        const uint32_t mB = ((s2 >> 4) & 0x0F0F0F0Fu) | ((s1 >> 2) & 0x30303030u);
        uint2 qh = make_uint2(0, 0);
        if constexpr (FMT == KQ_Q5_K) qh = lds8(L + Lay<KQ_Q5_K>::qh + r16 * Q5S + 8 * g);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint2 qv = lds8(qb + 32 * c);
            uint32_t lo0 = qv.x & 0x0F0F0F0Fu, lo1 = qv.y & 0x0F0F0F0Fu;
            uint32_t hi0 = (qv.x >> 4) & 0x0F0F0F0Fu, hi1 = (qv.y >> 4) & 0x0F0F0F0Fu;
            if constexpr (FMT == KQ_Q5_K) {
                // fifth bit of chunk j's weight 8g + e: bit j of high-bit byte 8g + e
                lo0 |= ((qh.x >> (2 * c)) & 0x01010101u) << 4;
                lo1 |= ((qh.y >> (2 * c)) & 0x01010101u) << 4;
                hi0 |= ((qh.x >> (2 * c + 1)) & 0x01010101u) << 4;
                hi1 |= ((qh.y >> (2 * c + 1)) & 0x01010101u) << 4;
            }
            const v4i D0 = mma_i8(lds8(cb + 64 * c), make_uint2(lo0, lo1));
            const v4i D1 = mma_i8(lds8(cb + 64 * c + 32), make_uint2(hi0, hi1));
            const uint32_t scw = c < 2 ? scA : scB;
            const int sc0 = (int)byte_of(scw, 2 * (c & 1)), sc1 = (int)byte_of(scw, 2 * (c & 1) + 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                P[i] += __mul24(sc0, D0[i]) + __mul24(sc1, D1[i]);
                asm volatile("" : "+v"(P[i]));  // one pair's operands live at a time
            }
        }
        // M = sum over bsums 4g .. 4g+3 (sub-blocks 2g, 2g, 2g+1, 2g+1) of m * bsum
        const uint32_t mw = g < 2 ? mA : mB;
        const float m0 = (float)byte_of(mw, 2 * (g & 1)), m1 = (float)byte_of(mw, 2 * (g & 1) + 1);
        v4h bm;
        bm[0] = (_Float16)m0;
        bm[1] = (_Float16)m0;
        bm[2] = (_Float16)m1;
        bm[3] = (_Float16)m1;
        const v4f Mv = mma_f16(ab, bm);
#pragma unroll
        for (int i = 0; i < 4; ++i) M[i] = Mv[i];
    }
}

}  // namespace

template <int FMT, bool PART>
__global__ __launch_bounds__(1024) void gemv_mma_kernel(const uint8_t *__restrict__ w, int64_t n, int nsb,
                                                        const int8_t *__restrict__ xq, const float *__restrict__ xs,
                                                        const int16_t *__restrict__ xbs, int T, float *__restrict__ y,
                                                        int32_t *__restrict__ Pout, int32_t *__restrict__ Mout,
                                                        int per_wave)
{
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kw = blockDim.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int64_t row0 = (int64_t)blockIdx.x * 16;
    const int64_t row = row0 + r16;
    const bool valid = row < n;
    const int64_t rows_left = n - row0;
    const Planes pl = planes_of(FMT, n, nsb);
    const int64_t rowsb0 = row0 * nsb;
    uint8_t *L = lds + wave * Lay<FMT>::size;
    float *red = reinterpret_cast<float *>(lds + kw * Lay<FMT>::size);  // [wave][half][token][row]
    // this lane's A-operand token: slot r16 (Q6_K: slot r16 & 7, see
    // superblock()); slots past the batch re-read the last token and feed
    // only output rows that are never stored
    const int ta = min(FMT == KQ_Q6_K ? (r16 & 7) : r16, T - 1);

    const int s_begin = wave * per_wave;
    const int s_end = min(nsb, s_begin + per_wave);
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};

    // Per superblock: stage the loads of s (waiting for them only: memory
    // counters retire in issue order), issue the loads of s + 1, fold s
    // from LDS while they stream in.
    Fetch<FMT> rw{};
    if (s_begin < s_end) fetch<FMT>(rw, w, pl, rowsb0, nsb, rows_left, s_begin, xq, xs, xbs, T, lane);
    for (int s = s_begin; s < s_end; ++s) {
        stage_lds<FMT>(rw, L, lane);
        const int sn = min(s + 1, s_end - 1);  // clamped: the last prefetch re-reads a valid superblock
        fetch<FMT>(rw, w, pl, rowsb0, nsb, rows_left, sn, xq, xs, xbs, T, lane);
        int P[4];
        float M[4], d, dmin;
        superblock<FMT>(L, r16, g, ta, P, M, d, dmin);
        const float4 d8v = reinterpret_cast<const float4 *>(L + Lay<FMT>::d)[g & 1];
        const float d8s[4] = {d8v.x, d8v.y, d8v.z, d8v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // tokens 4 (g & 1) + i: Q6_K lanes g and g ^ 2 hold the two
            // halves of one token's P; Q4_K/Q5_K lanes g >= 2 hold the
            // empty token slots 8..15
            const int t = 4 * (g & 1) + i;
            const float d8 = d8s[i];
            if (PART) {
                int Pt = P[i];
                if constexpr (FMT == KQ_Q6_K) Pt += __shfl_xor(P[i], 32);
                if (valid && t < T && g < 2) {
                    const int64_t o = ((int64_t)t * n + row) * nsb + s;
                    Pout[o] = Pt;
                    if (Mout) Mout[o] = (int)M[i];
                }
            }
            acc[i] = fmaf(d * d8, (float)P[i], acc[i]);
            if (FMT != KQ_Q6_K) acc[i] = fmaf(-(dmin * d8), M[i], acc[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wave * 2 + (g >> 1)) * TMAX + 4 * (g & 1) + i) * 16 + r16] = acc[i];
    __syncthreads();
    // the partial sums of each (token, row) in wave order (Q6_K: both halves
    // of each wave, first g < 2)
    for (int i = threadIdx.x; i < 16 * T; i += blockDim.x) {
        const int t = i >> 4, rl = i & 15;
        const int64_t rr = row0 + rl;
        if (rr < n) {
            float v = 0.0f;
            for (int kk = 0; kk < kw; ++kk) {
                v += red[((kk * 2) * TMAX + t) * 16 + rl];
                if constexpr (FMT == KQ_Q6_K) v += red[((kk * 2 + 1) * TMAX + t) * 16 + rl];
            }
            y[(int64_t)t * n + rr] = v;
        }
    }
}

// Batches 3..8 (the matrix core's 16 token slots hold up to 16).  The
// launch shape depends on n and k only, so the partials entry point sums in
// the same order.
int launch_gemv_mma(int fmt, const void *w, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                    const int16_t *xbs, int64_t t, float *y, int32_t *P, int32_t *M, hipStream_t st)
{
    if (t < 1 || t > TMAX) return KQ_EINVAL;
    const int64_t nsb = k / QK;
    const int64_t groups = (n + 15) / 16;
    // about 2048 waves over the chip, at most 16 per workgroup, every wave
    // of a workgroup with the same share of superblocks (2048 measured
    // fastest: 126.6 us against 129.7 us at 3072, summed over fourteen
    // Qwen3-4B FFN matrix and batch cases)
    int64_t nw = (2048 + groups - 1) / groups;
    nw = nw < 1 ? 1 : (nw > 16 ? 16 : nw);
    nw = nw > nsb ? nsb : nw;
    const int64_t per_wave = (nsb + nw - 1) / nw;
    const int64_t kw = (nsb + per_wave - 1) / per_wave;
    const dim3 g((unsigned)groups), b((unsigned)(64 * kw));
    const uint8_t *wp = (const uint8_t *)w;
    const bool part = P != nullptr;
    auto go = [&](auto fmtc) {
        constexpr int F = decltype(fmtc)::value;
        const size_t lds = (size_t)kw * Lay<F>::size + (size_t)kw * 2 * TMAX * 16 * sizeof(float);
        if (part)
            hipLaunchKernelGGL((gemv_mma_kernel<F, true>), g, b, lds, st, wp, n, (int)nsb, xq, xs, xbs, (int)t, y, P,
                               M, (int)per_wave);
        else
            hipLaunchKernelGGL((gemv_mma_kernel<F, false>), g, b, lds, st, wp, n, (int)nsb, xq, xs, xbs, (int)t, y,
                               P, M, (int)per_wave);
    };
    if (fmt == KQ_Q4_K) go(std::integral_constant<int, KQ_Q4_K>{});
    else if (fmt == KQ_Q5_K) go(std::integral_constant<int, KQ_Q5_K>{});
    else go(std::integral_constant<int, KQ_Q6_K>{});
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ELAUNCH;
}

}  // namespace kq
