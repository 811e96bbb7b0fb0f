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

template <typename T>
__device__ inline T ldg(const T *p) { return __builtin_nontemporal_load(p); }

}  // namespace kq
