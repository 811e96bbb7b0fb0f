// kq_pack.hip -- ggml superblock records <-> device planes (gfx950).
//
// The planes keep every byte of the records (the K-quant kernel arc page,
// "The pieces", kq v3 item: the DRAM planes keep the packed 160/192 B per
// superblock form, because decode time is plane bytes); they only regroup
// the fields so the matmul kernels issue aligned, coalesced 16-byte loads.
// The Q6_K record is 210 bytes, which no 16-byte load can walk in place.
// One thread per superblock; this runs once per weight matrix, at load.
#include "kq_common.h"

namespace kq {

// Field table: for each plane, the byte offset inside the record and the
// field length.  Planes are in the order of Planes::off.
struct Fields {
    int n;
    int rec_off[4];
    int len[4];
};

__host__ __device__ inline Fields fields_of(int fmt)
{
    if (fmt == KQ_Q4_K) return Fields{2, {0, 16, 0, 0}, {16, 128, 0, 0}};
    if (fmt == KQ_Q5_K) return Fields{3, {0, 16, 48, 0}, {16, 32, 128, 0}};
    return Fields{4, {0, 128, 192, 208}, {128, 64, 16, 2}};  // Q6_K
}

template <bool TO_PLANES>
__global__ __launch_bounds__(256) void pack_kernel(int fmt, const uint8_t *__restrict__ src,
                                                   uint8_t *__restrict__ dst, int64_t S, int64_t n,
                                                   int64_t nsb)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= S) return;
    const Planes p = planes_of(fmt, n, nsb);
    const Fields f = fields_of(fmt);
    const int rb = record_bytes(fmt);
    for (int q = 0; q < f.n; ++q) {
        const int len = f.len[q];
        const uint8_t *rec_field = (TO_PLANES ? src : dst) + i * rb + f.rec_off[q];
        const uint8_t *plane_field = (TO_PLANES ? dst : src) + p.off[q] + i * len;
        const uint8_t *from = TO_PLANES ? rec_field : plane_field;
        uint8_t *to = const_cast<uint8_t *>(TO_PLANES ? plane_field : rec_field);
        if (fmt != KQ_Q6_K) {
            // Q4_K/Q5_K records are 144/176 B: every field is 16-byte aligned
            for (int b = 0; b < len; b += 16)
                *reinterpret_cast<uint4 *>(to + b) = *reinterpret_cast<const uint4 *>(from + b);
        } else {
            for (int b = 0; b < len; ++b) to[b] = from[b];
        }
    }
}

static int launch_pack_common(bool to_planes, int fmt, const void *src, int64_t n, int64_t k, void *dst,
                              hipStream_t stream)
{
    const int64_t nsb = k / QK, S = n * nsb;
    const int64_t blocks = (S + 255) / 256;
    if (to_planes)
        hipLaunchKernelGGL(pack_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, fmt,
                           (const uint8_t *)src, (uint8_t *)dst, S, n, nsb);
    else
        hipLaunchKernelGGL(pack_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, fmt,
                           (const uint8_t *)src, (uint8_t *)dst, S, n, nsb);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ELAUNCH;
}

int launch_pack(int fmt, const void *w_ggml, int64_t n, int64_t k, void *w_planes, hipStream_t stream)
{
    return launch_pack_common(true, fmt, w_ggml, n, k, w_planes, stream);
}

int launch_unpack(int fmt, const void *w_planes, int64_t n, int64_t k, void *w_ggml, hipStream_t stream)
{
    return launch_pack_common(false, fmt, w_planes, n, k, w_ggml, stream);
}

}  // namespace kq
