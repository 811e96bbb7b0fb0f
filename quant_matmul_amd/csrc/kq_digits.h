// kq_digits.h -- the GEMMs' operand form of a K-quant weight: the
// sub-scale-folded value w' = sc*q (Q4_K/Q5_K) or sc*(q-32) (Q6_K), split
// into two int8 digits, four weights per dword: w' = 128*h + l, l in 0..127
// (Q5_K, Q6_K), or w' = 8*(u*q) + (v*q) with sc = 8u + v (Q4_K).  The int8
// MFMA then forms the per-sub-block integer fold P = sum sc*dot as
// 2^SHIFT*(h . a) + (l . a) (K-quant kernel arc page, "The pieces", kq v2
// item).
#pragma once

#include "kq_common.h"

namespace kq {
namespace {

// byte selectors of v_perm_b32 (bytes 0..3 = second operand, 4..7 = first)
constexpr uint32_t SEL_EVEN = 0x0C020C00u;    // bytes 0, 2 -> 16-bit lanes
constexpr uint32_t SEL_ODD = 0x0C030C01u;     // bytes 1, 3 -> 16-bit lanes
constexpr uint32_t SEL_INTERLEAVE = 0x06020400u;  // low bytes of (e, o) lanes -> e0 o0 e1 o1

// Digits of four 16-bit lane values (e = v0 | v2 << 16, o = v1 | v3 << 16,
// each in [0, 16383]): low digits (bits 0..6) and high digits (bits 7..13)
// packed as bytes v0 v1 v2 v3.  (e >> 7) keeps each lane's bits 7..14 in
// that lane's low byte: the upper lane's bits move to bit 9 and up.
__device__ inline void split_digits(uint32_t e, uint32_t o, uint32_t &hi, uint32_t &lo)
{
    lo = __builtin_amdgcn_perm(o, e, SEL_INTERLEAVE) & 0x7F7F7F7Fu;
    hi = __builtin_amdgcn_perm(o >> 7, e >> 7, SEL_INTERLEAVE);
}

// Four unsigned quants (one per byte of q, each <= 31) times scale sc
// (0..63): the digits of sc*q.
__device__ inline void digits_q45(uint32_t q, int sc, uint32_t &hi, uint32_t &lo)
{
    // each 16-bit lane <= 31*63, and both factors fit 24 bits
    const uint32_t e = (uint32_t)__umul24(__builtin_amdgcn_perm(0u, q, SEL_EVEN), (uint32_t)sc);
    const uint32_t o = (uint32_t)__umul24(__builtin_amdgcn_perm(0u, q, SEL_ODD), (uint32_t)sc);
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
    const uint32_t e = (uint32_t)(__mul24((int)__builtin_amdgcn_perm(0u, q, SEL_EVEN), sc) + bias);
    const uint32_t o = (uint32_t)(__mul24((int)__builtin_amdgcn_perm(0u, q, SEL_ODD), sc) + bias);
    uint32_t hu;
    split_digits(e, o, hu, lo);
    hi = ((hu | 0x80808080u) - 0x20202020u) ^ 0x80808080u;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Q4_K's other split.  Its quants are 4-bit, so with the sub-scale written
// as sc = 8*u + v (u, v in 0..7) both u*q and v*q are at most 105: they fit
// a signed byte and four of them come out of one packed 16-bit multiply
// with no carry between bytes.  Then sc*q = 8*(u*q) + (v*q), and the two
// MFMA passes give P = 8*H + L.  Four quants (bytes of q, each <= 15):
__device__ inline void digits_q4(uint32_t q, int u, int v, uint32_t &hi, uint32_t &lo)
{
    const u16x2 qq = __builtin_bit_cast(u16x2, q);
    hi = __builtin_bit_cast(uint32_t, qq * u16x2{(unsigned short)u, (unsigned short)u});
    lo = __builtin_bit_cast(uint32_t, qq * u16x2{(unsigned short)v, (unsigned short)v});
}

}  // namespace
}  // namespace kq
