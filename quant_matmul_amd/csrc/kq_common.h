// kq_common.h -- internal helpers shared by the kq HIP kernels (gfx950).
//
// Device planes.  kq_pack splits each format's superblock records by field
// into separate row-major planes, each starting on a 256-byte boundary:
//
//   Q4_K  hdr[S][16]  (f16 d, f16 dmin, 12 B 6-bit scale/min packing)
//         qs [S][128] (4-bit quants)
//   Q5_K  hdr[S][16], qh[S][32] (fifth bits), qs[S][128]
//   Q6_K  ql [S][128] (low 4 bits), qh[S][64] (high 2 bits),
//         sc [S][16]  (int8 scale per 16 weights), d[S] (f16)
//
// with S = n * (k/256) superblocks in row-major [row][superblock] order.  The
// bytes are the ggml record bytes, only regrouped, so every 16-byte load of a
// plane is aligned and a quad of lanes reads whole cache lines.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq.h"

namespace kq {

constexpr int QK = 256;
// largest k the GEMM takes: 256 tokens of codes stay below 2^31 bytes
constexpr int64_t GEMM_KMAX = ((int64_t)1 << 23) - QK;

__host__ __device__ inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

struct Planes {
    int64_t off[4];  // byte offset of each plane from the planes base
    int64_t total;   // total bytes
};

__host__ __device__ inline Planes planes_of(int fmt, int64_t n, int64_t nsb)
{
    const int64_t S = n * nsb;
    Planes p{{0, 0, 0, 0}, 0};
    if (fmt == KQ_Q4_K) {
        p.off[0] = 0;                       // hdr
        p.off[1] = align256(16 * S);        // qs
        p.total = p.off[1] + align256(128 * S);
    } else if (fmt == KQ_Q5_K) {
        p.off[0] = 0;                       // hdr
        p.off[1] = align256(16 * S);        // qh
        p.off[2] = p.off[1] + align256(32 * S);  // qs
        p.total = p.off[2] + align256(128 * S);
    } else if (fmt == KQ_Q6_K) {
        p.off[0] = 0;                       // ql
        p.off[1] = align256(128 * S);       // qh
        p.off[2] = p.off[1] + align256(64 * S);  // sc
        p.off[3] = p.off[2] + align256(16 * S);  // d
        p.total = p.off[3] + align256(2 * S);
    }
    return p;
}

__host__ __device__ inline int record_bytes(int fmt)
{
    return fmt == KQ_Q4_K ? 144 : fmt == KQ_Q5_K ? 176 : fmt == KQ_Q6_K ? 210 : 0;
}

// --------------------------------------------------------------- device --
__device__ inline float f16_bits_to_float(uint32_t h16)
{
    // binary16 -> binary32 through the hardware conversion (exact; f16
    // subnormals are normal binary32 numbers)
    _Float16 h;
    uint16_t b = (uint16_t)h16;
    __builtin_memcpy(&h, &b, 2);
    return (float)h;
}

__device__ inline int sdot4(int a, int b, int c) { return __builtin_amdgcn_sdot4(a, b, c, false); }

// Byte i (0..3, runtime) of a dword.
__device__ inline uint32_t byte_of(uint32_t w, int i) { return (w >> (8 * i)) & 0xFFu; }

// The 6-bit scale and min of sub-block j (0..7) from the 12-byte packing
// held in three dwords s0 = bytes 0..3, s1 = bytes 4..7, s2 = bytes 8..11:
//   j < 4:  sc = byte j & 63,            m = byte j+4 & 63
//   j >= 4: sc = (byte j+4 & 15) | (byte j-4 >> 6) << 4
//           m  = (byte j+4 >> 4) | (byte j >> 6) << 4
__device__ inline void scale_min_6bit(uint32_t s0, uint32_t s1, uint32_t s2, int j, int &sc, int &m)
{
    const int jl = j & 3;
    const uint32_t b0 = byte_of(s0, jl), b1 = byte_of(s1, jl), b2 = byte_of(s2, jl);
    const int lo_sc = b0 & 63, lo_m = b1 & 63;
    const int hi_sc = (b2 & 15) | ((b0 >> 6) << 4);
    const int hi_m = (b2 >> 4) | ((b1 >> 6) << 4);
    sc = j < 4 ? lo_sc : hi_sc;
    m = j < 4 ? lo_m : hi_m;
}

// Sum over the 4 lanes of a quad (lanes 4i..4i+3), result in every lane.
__device__ inline int quad_sum(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    return v;
}

// Q8_K codes.  The code of x is rint(x / d8), the correctly rounded binary32
// quotient rounded half to even, clamped to [-127, 127].  The quotient is
// formed without a full IEEE division per value (Markstein's method, as in
// the IA-64 division sequences): with y = 1/d8 correctly rounded,
// q0 = x*y is within a few ulps of x/d8, and each correction
// q += (x - q*d8)*y, whose residual one fma gives exactly, brings q closer;
// after two corrections q is the correctly rounded quotient.  That needs
// the residuals to stay in the normal range wherever the code can be
// nonzero (|x| >= d8/2), which d8 >= 2^-64 guarantees; a chunk with a
// smaller scale (amax below about 2^-57) takes the IEEE division
// (__fdiv_rn) per value instead.  1/d8 cannot overflow for d8 >= 2^-64,
// and d8 <= amax/127 keeps every product in range.
__device__ inline float q8k_recip(float d8) { return d8 >= 0x1p-64f ? __fdiv_rn(1.0f, d8) : 0.0f; }

__device__ inline int q8k_code(float x, float d8, float y)
{
    float q;
    if (y != 0.0f) {
        q = x * y;
        q = fmaf(fmaf(-q, d8, x), y, q);
        q = fmaf(fmaf(-q, d8, x), y, q);
    } else {
        q = __fdiv_rn(x, d8);
    }
    const int a = (int)rintf(q);
    return a > 127 ? 127 : (a < -127 ? -127 : a);
}

template <int CTRL>
__device__ inline float dpp_max(float v)
{
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false)));
}

// Maximum over each row of 16 lanes, in every lane of the row (max is exact,
// so any order gives the same bits).
__device__ inline float row_max(float v)
{
    v = dpp_max<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_max<0x4E>(v);   // quad_perm [2,3,0,1]
    v = dpp_max<0x141>(v);  // row_half_mirror
    return dpp_max<0x140>(v);  // row_mirror
}

// Maximum over the 64 lanes: the four row maxima.
__device__ inline float wave_max(float v)
{
    v = row_max(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Q8_K quantisation of one 256-value chunk by one wave: lane l holds values
// 4l..4l+3.  amax over the chunk, d8 = amax/127 (binary32, correctly
// rounded), codes as above; an all-zero chunk gives d8 = 0 and zero codes.
// Returns the lane's four codes packed in a dword; `qsum` receives the sum
// of the 16 codes of the lane's quad (bsum g = l/4) and d8 the scale.
__device__ inline uint32_t q8k_chunk(float4 v, int &qsum, float &d8)
{
    const float amax = wave_max(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
    d8 = 0.0f;
    if (amax != 0.0f) {
        d8 = __fdiv_rn(amax, 127.0f);
        const float y = q8k_recip(d8);
        a0 = q8k_code(v.x, d8, y);
        a1 = q8k_code(v.y, d8, y);
        a2 = q8k_code(v.z, d8, y);
        a3 = q8k_code(v.w, d8, y);
    }
    qsum = quad_sum(a0 + a1 + a2 + a3);
    return (uint32_t)(a0 & 0xFF) | ((uint32_t)(a1 & 0xFF) << 8) | ((uint32_t)(a2 & 0xFF) << 16) |
           ((uint32_t)(a3 & 0xFF) << 24);
}

// Q8_K quantisation of four chunks by one wave (the wide form): the 16 lanes
// of row r each hold 16 consecutive values v[0..15] of one chunk, lane j of
// the row values 16j..16j+15.  All 64 lanes must be active (the amax is a
// DPP reduction over the row).  Returns the lane's 16 codes as one 16-byte
// piece; `qsum` receives their sum (bsum j of the chunk) and d8 the
// chunk's scale.
__device__ inline uint4 q8k_piece16(const float (&v)[16], int &qsum, float &d8)
{
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = row_max(amax);
    uint32_t pk[4] = {0, 0, 0, 0};
    qsum = 0;
    d8 = 0.0f;
    if (amax != 0.0f) {
        d8 = __fdiv_rn(amax, 127.0f);
        const float y = q8k_recip(d8);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int a = q8k_code(v[i], d8, y);
            qsum += a;
            pk[i >> 2] |= (uint32_t)(a & 0xFF) << (8 * (i & 3));
        }
    }
    return make_uint4(pk[0], pk[1], pk[2], pk[3]);
}

// Raw bytes of one 64-weight share of a superblock, as loaded from the
// planes by one lane (GEMV) or one unpack task (GEMM), before any compute.
// Share c of a Q4_K/Q5_K superblock is sub-blocks 2c and 2c+1 (the low and
// high nibbles of quant bytes 32c..32c+31); share c = 2h + u of a Q6_K
// superblock is the low-array bytes 64h + 32u .. +31 (weights 128h + 32u +
// 0..31 and + 64 + 0..31), their high-bit bytes and their four scales.
template <int FMT>
struct Raw;
template <>
struct Raw<KQ_Q4_K> {
    uint4 h, q0, q1;
};
template <>
struct Raw<KQ_Q5_K> {
    uint4 h, q0, q1, qh0, qh1;
};
template <>
struct Raw<KQ_Q6_K> {
    uint4 l0, l1, h0, h1;
    uint2 s8;
    uint32_t d;
};

// Q4_K / Q5_K: lane c covers sub-blocks 2c (low nibbles of quant bytes
// 32c..32c+31) and 2c+1 (their high nibbles).
__device__ inline void load_raw(Raw<KQ_Q4_K> &r, const uint8_t *__restrict__ w, const Planes &pl, int64_t sb, int c)
{
    r.h = *reinterpret_cast<const uint4 *>(w + pl.off[0] + sb * 16);
    const uint4 *qs = reinterpret_cast<const uint4 *>(w + pl.off[1] + sb * 128 + 32 * c);
    r.q0 = qs[0];
    r.q1 = qs[1];
}
__device__ inline void load_raw(Raw<KQ_Q5_K> &r, const uint8_t *__restrict__ w, const Planes &pl, int64_t sb, int c)
{
    r.h = *reinterpret_cast<const uint4 *>(w + pl.off[0] + sb * 16);
    const uint4 *qh = reinterpret_cast<const uint4 *>(w + pl.off[1] + sb * 32);
    r.qh0 = qh[0];
    r.qh1 = qh[1];
    const uint4 *qs = reinterpret_cast<const uint4 *>(w + pl.off[2] + sb * 128 + 32 * c);
    r.q0 = qs[0];
    r.q1 = qs[1];
}
// Q6_K: lane c = 2h + u covers the low-array bytes 64h + 32u .. +31.
__device__ inline void load_raw(Raw<KQ_Q6_K> &r, const uint8_t *__restrict__ w, const Planes &pl, int64_t sb, int c)
{
    const int h = c >> 1, u = c & 1;
    const uint4 *ql = reinterpret_cast<const uint4 *>(w + pl.off[0] + sb * 128 + 64 * h + 32 * u);
    const uint4 *qh = reinterpret_cast<const uint4 *>(w + pl.off[1] + sb * 64 + 32 * h);
    r.l0 = ql[0];
    r.l1 = ql[1];
    r.h0 = qh[0];
    r.h1 = qh[1];
    r.s8 = *reinterpret_cast<const uint2 *>(w + pl.off[2] + sb * 16 + 8 * h);
    r.d = *reinterpret_cast<const uint16_t *>(w + pl.off[3] + sb * 2);
}

}  // namespace kq
