// kq_gemv.hip -- decode GEMV, batch 1..8 (gfx950): batches 1-2 here, on
// packed int8 dot instructions; batches 3-8 on the matrix cores
// (kq_gemv_mma.hip), where the per-token dot work would dominate.
//
// y[t][n] = sum_s fold(P, M) over superblocks s (K-quant kernel arc page,
// "The pieces", kq v2 item; k4 v2 and k5/k6 v2 commit messages): the
// sub-scale x int32 dot and min x bsum terms are accumulated in int32 per
// superblock and closed by ONE float fold per (token, row, superblock).
//
// Work mapping.  A quad of lanes owns one superblock of one row; lane c of
// the quad owns 64 consecutive-in-record weights (two sub-blocks for Q4_K /
// Q5_K, four 16-wide sub-blocks for Q6_K), loads its 32 bytes of 4-bit
// quants (plus its high bits) with 16-byte loads, unpacks them in registers
// and dots them with sdot4 against the Q8_K codes.  The quad's four int32
// partials are summed with two DPP steps, so every lane of the quad holds
// the superblock's exact P (and M); the float fold follows.  A wave covers
// 16 rows at one superblock per step; the waves of a workgroup share the
// same 16 rows and split the superblocks between them, and their float sums
// meet in LDS.  Decode streams the weight planes exactly once (the page's
// "decode reads the whole blob per token", kq v3 commit message).
#include <type_traits>

#include "kq_common.h"

namespace kq {

namespace {

struct Lane {
    int p, m;  // this lane's share of P and M for one token
};

// The Q8_K codes and bsums one lane dots against its 64 weights, for one
// token of one superblock (a: the token's codes of the superblock, bs: its
// 16 bsums).
struct Act {
    uint4 a0, a1, a2, a3;
    uint4 b;
};

template <int FMT>
__device__ inline void load_act(Act &r, const int8_t *__restrict__ a, const int16_t *__restrict__ bs, int c)
{
    if constexpr (FMT == KQ_Q6_K) {
        // codes 128h + 32u + 0..31 and + 64; bsums 8h..8h+7
        const int h = c >> 1, u = c & 1;
        const uint4 *at = reinterpret_cast<const uint4 *>(a + 128 * h + 32 * u);
        r.a0 = at[0];
        r.a1 = at[1];
        r.a2 = at[4];
        r.a3 = at[5];
        r.b = *reinterpret_cast<const uint4 *>(bs + 8 * h);
    } else {
        // codes 64c..64c+63; bsums 4c..4c+3
        const uint4 *ap = reinterpret_cast<const uint4 *>(a + 64 * c);
        r.a0 = ap[0];
        r.a1 = ap[1];
        r.a2 = ap[2];
        r.a3 = ap[3];
        const uint2 b = *reinterpret_cast<const uint2 *>(bs + 4 * c);
        r.b = make_uint4(b.x, b.y, 0, 0);
    }
}

template <int FMT, int T>
__device__ inline void compute_q45(const Raw<FMT> &r, int c, const Act (&act)[T], Lane (&out)[T], float &d,
                                   float &dmin)
{
    uint32_t lo[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
    uint32_t hi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        hi[i] = (lo[i] >> 4) & 0x0F0F0F0Fu;
        lo[i] &= 0x0F0F0F0Fu;
    }
    if constexpr (FMT == KQ_Q5_K) {
        // fifth bit of weight 32j + l is bit j of high-bit byte l
        const uint32_t hb[8] = {r.qh0.x, r.qh0.y, r.qh0.z, r.qh0.w, r.qh1.x, r.qh1.y, r.qh1.z, r.qh1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            lo[i] |= ((hb[i] >> (2 * c)) & 0x01010101u) << 4;
            hi[i] |= ((hb[i] >> (2 * c + 1)) & 0x01010101u) << 4;
        }
    }
    d = f16_bits_to_float(r.h.x & 0xFFFFu);
    dmin = f16_bits_to_float(r.h.x >> 16);
    int sc0, m0, sc1, m1;
    scale_min_6bit(r.h.y, r.h.z, r.h.w, 2 * c, sc0, m0);
    scale_min_6bit(r.h.y, r.h.z, r.h.w, 2 * c + 1, sc1, m1);
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const uint4 A0 = act[t].a0, A1 = act[t].a1, A2 = act[t].a2, A3 = act[t].a3;
        int dl = 0, dh = 0;
        dl = sdot4(lo[0], A0.x, dl); dl = sdot4(lo[1], A0.y, dl);
        dl = sdot4(lo[2], A0.z, dl); dl = sdot4(lo[3], A0.w, dl);
        dl = sdot4(lo[4], A1.x, dl); dl = sdot4(lo[5], A1.y, dl);
        dl = sdot4(lo[6], A1.z, dl); dl = sdot4(lo[7], A1.w, dl);
        dh = sdot4(hi[0], A2.x, dh); dh = sdot4(hi[1], A2.y, dh);
        dh = sdot4(hi[2], A2.z, dh); dh = sdot4(hi[3], A2.w, dh);
        dh = sdot4(hi[4], A3.x, dh); dh = sdot4(hi[5], A3.y, dh);
        dh = sdot4(hi[6], A3.z, dh); dh = sdot4(hi[7], A3.w, dh);
        // bsums 4c..4c+3: the first two cover sub-block 2c, the last two 2c+1
        const uint2 b = make_uint2(act[t].b.x, act[t].b.y);
        const int b0 = (int16_t)(b.x & 0xFFFF), b1 = (int16_t)(b.x >> 16);
        const int b2 = (int16_t)(b.y & 0xFFFF), b3 = (int16_t)(b.y >> 16);
        out[t].p = sc0 * dl + sc1 * dh;
        out[t].m = m0 * (b0 + b1) + m1 * (b2 + b3);
    }
}

// Q6_K lane c = 2h + u: the low nibbles of its 32 low-array bytes are
// weights 128h + 32u + l (16-wide sub-blocks 8h+2u, 8h+2u+1), the high
// nibbles weights 128h + 32u + 64 + l (sub-blocks 8h+2u+4, 8h+2u+5); the
// high two bits come from bits 2u.. (resp. 2u+4..) of high byte 32h + l.
// Signed scales; P = iacc - 32*bacc, exact in int32.
template <int T>
__device__ inline void compute_q6(const Raw<KQ_Q6_K> &r, int c, const Act (&act)[T], Lane (&out)[T], float &d)
{
    const int h = c >> 1, u = c & 1;
    const uint32_t lw[8] = {r.l0.x, r.l0.y, r.l0.z, r.l0.w, r.l1.x, r.l1.y, r.l1.z, r.l1.w};
    const uint32_t hw[8] = {r.h0.x, r.h0.y, r.h0.z, r.h0.w, r.h1.x, r.h1.y, r.h1.z, r.h1.w};
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        lo[i] = (lw[i] & 0x0F0F0F0Fu) | (((hw[i] >> (2 * u)) & 0x03030303u) << 4);
        hi[i] = ((lw[i] >> 4) & 0x0F0F0F0Fu) | (((hw[i] >> (2 * u + 4)) & 0x03030303u) << 4);
    }
    d = f16_bits_to_float(r.d);
    const int sa = (int8_t)byte_of(r.s8.x, 2 * u), sb_ = (int8_t)byte_of(r.s8.x, 2 * u + 1);
    const int sc_ = (int8_t)byte_of(r.s8.y, 2 * u), sd = (int8_t)byte_of(r.s8.y, 2 * u + 1);
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const uint4 A0 = act[t].a0, A1 = act[t].a1, A2 = act[t].a2, A3 = act[t].a3;
        int d0 = 0, d1 = 0, d2 = 0, d3 = 0;
        d0 = sdot4(lo[0], A0.x, d0); d0 = sdot4(lo[1], A0.y, d0);
        d0 = sdot4(lo[2], A0.z, d0); d0 = sdot4(lo[3], A0.w, d0);
        d1 = sdot4(lo[4], A1.x, d1); d1 = sdot4(lo[5], A1.y, d1);
        d1 = sdot4(lo[6], A1.z, d1); d1 = sdot4(lo[7], A1.w, d1);
        d2 = sdot4(hi[0], A2.x, d2); d2 = sdot4(hi[1], A2.y, d2);
        d2 = sdot4(hi[2], A2.z, d2); d2 = sdot4(hi[3], A2.w, d2);
        d3 = sdot4(hi[4], A3.x, d3); d3 = sdot4(hi[5], A3.y, d3);
        d3 = sdot4(hi[6], A3.z, d3); d3 = sdot4(hi[7], A3.w, d3);
        // bsums 8h..8h+7: 2u, 2u+1 pair with the low half, 2u+4, 2u+5 the high
        const uint4 b = act[t].b;
        const uint32_t blo = u ? b.y : b.x, bhi = u ? b.w : b.z;
        const int ba = (int16_t)(blo & 0xFFFF), bb = (int16_t)(blo >> 16);
        const int bc = (int16_t)(bhi & 0xFFFF), bd = (int16_t)(bhi >> 16);
        const int iacc = sa * d0 + sb_ * d1 + sc_ * d2 + sd * d3;
        const int bacc = sa * ba + sb_ * bb + sc_ * bc + sd * bd;
        out[t].p = iacc - 32 * bacc;
        out[t].m = 0;
    }
}

}  // namespace

template <int CTRL>
__device__ inline float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// One workgroup = RGS row groups of 16/SL rows x all superblocks.  A wave
// step covers SL adjacent superblocks of each of its group's 16/SL rows
// (quad q = sig + SL*rho of the wave: superblock slot sig, row rho), so
// small-n matrices still spread over many waves; the kw waves of a row
// group take contiguous runs of `per_wave` steps, one step's weight loads
// in flight at a time (two steps' loads per wave measured 2-4% slower on
// the 14-73 MB matrices, three or five slower still).  The SL
// slot sums of a row meet by DPP mirrors, the kw waves' sums in LDS.  The
// activation image is staged (or, fused, quantised) once per workgroup, so
// a workgroup of several row groups pays for it once.
//
// FUSE (batch <= 2): the workgroup quantises the f32 activation x itself
// into its LDS stage (the same per-chunk arithmetic as kq_quantize_q8k, so
// the image is bit-identical) instead of reading a Q8_K image; workgroup 0
// also writes that image out when oq is non-null.
template <int FMT, int T, int SL, bool PART, bool FUSE, bool STG, int SMAX>
__global__ __launch_bounds__(1024) void gemv_kernel(const uint8_t *__restrict__ w, int64_t n, int nsb,
                                                    const int8_t *__restrict__ xq, const float *__restrict__ xs,
                                                    const int16_t *__restrict__ xbs, float *__restrict__ y,
                                                    int32_t *__restrict__ Pout, int32_t *__restrict__ Mout,
                                                    int per_wave, int kw, const float *__restrict__ x,
                                                    int8_t *__restrict__ oq, float *__restrict__ os,
                                                    int16_t *__restrict__ obs)
{
    static_assert(T <= 2, "batches past 2 run on the matrix cores");
    static_assert(!FUSE || STG, "the fused quantiser stages the image in LDS");
    constexpr int RPW = 16 / SL;
    __shared__ float red[16][T][RPW];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int c = lane & 3, quad = lane >> 2;
    const int sig = quad % SL, rho = quad / SL;
    // several row groups per workgroup only when fused (the plain GEMV runs
    // one, and keeps its first weight loads free of the division)
    const int rgs = FUSE ? nw / kw : 1, rgi = FUSE ? wave / kw : 0, kwi = FUSE ? wave - rgi * kw : wave;
    const int64_t row = ((int64_t)blockIdx.x * rgs + rgi) * RPW + rho;
    const bool valid = row < n;
    const int64_t K = (int64_t)nsb * QK, KB = K / 16;
    const Planes pl = planes_of(FMT, n, nsb);
    // rows past n read row 0 (in bounds) and are never stored
    const int64_t rbase = (valid ? row : 0) * nsb;

    float acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.0f;

    const int nsteps = (nsb + SL - 1) / SL;
    const int j_begin = kwi * per_wave;
    const int j_end = min(nsteps, j_begin + per_wave);
    // this lane's superblock at step j, clamped in bounds (out-of-range
    // slots re-read a valid superblock and contribute nothing)
    auto sb_at = [&](int j) { return min(min(j, j_end - 1) * SL + sig, nsb - 1); };

    // STG: the whole Q8_K image (codes + bsums, T*K*9/8 bytes) is staged in
    // LDS with coalesced 16-byte loads, so no lane waits on an L2 round trip
    // for its codes after its weights land (while it fits: k up to about
    // 128k; longer rows read the codes straight from L2 inside the loop).
    // Memory counters retire in issue order, so the staging loads go out
    // before the weight loads: writing them to LDS then waits only for
    // themselves, and their L2 latency hides under the HBM fetch of the
    // weights.  SMAX chunks per thread go out ahead of the weights (2, or 6
    // when the image holds more than two per thread: the long rows of the
    // large dense matrices); the rest follow them.
    constexpr bool LDSA = STG;
    extern __shared__ __align__(16) uint8_t stage[];
    const int64_t nq = T * K / 16, nst = nq + T * K / 128;  // chunks: codes, then bsums
    auto src_chunk = [&](int64_t i) {
        return i < nq ? reinterpret_cast<const uint4 *>(xq)[i] : reinterpret_cast<const uint4 *>(xbs)[i - nq];
    };
    uint4 st[SMAX];
    if constexpr (LDSA && !FUSE) {
#pragma unroll
        for (int j = 0; j < SMAX; ++j) {
            const int64_t i = threadIdx.x + (int64_t)j * blockDim.x;
            if (i < nst) st[j] = src_chunk(i);
        }
    }
    // fused: the activation's chunks (chunk = t*nsb + s) are quantised four
    // per wave, in groups g = 4 consecutive chunks: wave w takes groups w,
    // w + nw, ...; lane l holds values 16j..16j+15 (j = l % 16) of chunk
    // 4g + l/16.  The first GMAX groups of a wave are loaded before the
    // weights.
    constexpr int GMAX = 2;
    const int nchunks = T * nsb, ngroups = (nchunks + 3) >> 2;
    const int gsub = lane >> 4, gj = lane & 15;
    auto load_group = [&](int g, float (&v)[16]) {
        const int ch = 4 * g + gsub;
        const float4 *p = reinterpret_cast<const float4 *>(x + (int64_t)ch * QK + 16 * gj);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 f = ch < nchunks ? p[i] : make_float4(0, 0, 0, 0);
            v[4 * i] = f.x;
            v[4 * i + 1] = f.y;
            v[4 * i + 2] = f.z;
            v[4 * i + 3] = f.w;
        }
    };
    float xv[FUSE ? GMAX : 1][16];
    if constexpr (FUSE) {
#pragma unroll
        for (int gi = 0; gi < GMAX; ++gi)
            if (wave + gi * nw < ngroups) load_group(wave + gi * nw, xv[gi]);
    }

    // unconditional, so the count of loads in flight is static and the
    // staging write below waits only for the staging loads
    Raw<FMT> raw;
    load_raw(raw, w, pl, rbase + sb_at(j_begin), c);

    const int8_t *aq = xq;
    const int16_t *ab = xbs;
    const float *d8src = xs;
    if constexpr (FUSE) {
        int8_t *sq = reinterpret_cast<int8_t *>(stage);
        int16_t *sbs = reinterpret_cast<int16_t *>(stage + T * K);
        float *sd8 = reinterpret_cast<float *>(stage + T * K * 9 / 8);
        // every lane of the wave runs the quantiser (its amax is a DPP row
        // reduction); rows past the last chunk hold zeros and store nothing
        auto quant = [&](int g, const float (&v)[16]) {
            const int ch = 4 * g + gsub;
            int qsum;
            float d8;
            const uint4 piece = q8k_piece16(v, qsum, d8);
            if (ch < nchunks) {
                reinterpret_cast<uint4 *>(sq + (int64_t)ch * QK)[gj] = piece;
                sbs[ch * 16 + gj] = (int16_t)qsum;
                if (gj == 0) sd8[ch] = d8;
            }
        };
#pragma unroll
        for (int gi = 0; gi < GMAX; ++gi)
            if (wave + gi * nw < ngroups) quant(wave + gi * nw, xv[gi]);
        for (int g = wave + GMAX * nw; g < ngroups; g += nw) {
            float v[16];
            load_group(g, v);
            quant(g, v);
        }
        __syncthreads();
        if (oq != nullptr && blockIdx.x == 0) {
            // the Q8_K image, for callers that keep it
            for (int64_t i = threadIdx.x; i < T * K / 16; i += blockDim.x)
                reinterpret_cast<uint4 *>(oq)[i] = reinterpret_cast<const uint4 *>(sq)[i];
            for (int64_t i = threadIdx.x; i < T * K / 128; i += blockDim.x)
                reinterpret_cast<uint4 *>(obs)[i] = reinterpret_cast<const uint4 *>(sbs)[i];
            for (int i = threadIdx.x; i < nchunks; i += blockDim.x) os[i] = sd8[i];
        }
        aq = sq;
        ab = sbs;
        d8src = sd8;
    } else if constexpr (LDSA) {
        uint4 *dst = reinterpret_cast<uint4 *>(stage);
#pragma unroll
        for (int j = 0; j < SMAX; ++j) {
            const int64_t i = threadIdx.x + (int64_t)j * blockDim.x;
            if (i < nst) dst[i] = st[j];
        }
        for (int64_t i = threadIdx.x + (int64_t)SMAX * blockDim.x; i < nst; i += blockDim.x) dst[i] = src_chunk(i);
        __syncthreads();
        aq = reinterpret_cast<const int8_t *>(stage);
        ab = reinterpret_cast<const int16_t *>(stage + T * K);
    }

    for (int j = j_begin; j < j_end; ++j) {
        if (j != j_begin) load_raw(raw, w, pl, rbase + sb_at(j), c);
        const int s = sb_at(j);
        const bool live = j * SL + sig < nsb;  // slot holds a real superblock
        Act cur[T];
#pragma unroll
        for (int t = 0; t < T; ++t)
            load_act<FMT>(cur[t], aq + t * K + (int64_t)s * QK, ab + t * KB + (int64_t)s * 16, c);
        Lane part[T];
        float d, dmin = 0.0f;
        if constexpr (FMT == KQ_Q6_K)
            compute_q6<T>(raw, c, cur, part, d);
        else
            compute_q45<FMT, T>(raw, c, cur, part, d, dmin);
        d = live ? d : 0.0f;
        dmin = live ? dmin : 0.0f;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            // DPP sums run with every lane of the wave active
            const int P = quad_sum(part[t].p);
            const int M = FMT == KQ_Q6_K ? 0 : quad_sum(part[t].m);
            const float d8 = d8src[t * nsb + s];
            if (PART && c == 0 && valid && live) {
                const int64_t o = ((int64_t)t * n + row) * nsb + s;
                Pout[o] = P;
                if (Mout) Mout[o] = M;
            }
            acc[t] = fmaf(d * d8, (float)P, acc[t]);
            if (FMT != KQ_Q6_K) acc[t] = fmaf(-(dmin * d8), (float)M, acc[t]);
        }
    }

    // sum the SL superblock slots of each row (identical across a quad)
#pragma unroll
    for (int t = 0; t < T; ++t) {
        if constexpr (SL >= 2) acc[t] += dpp_f<0x141>(acc[t]);  // row_half_mirror: quad pairs
        if constexpr (SL >= 4) acc[t] += dpp_f<0x140>(acc[t]);  // row_mirror: quad 0<->3, 1<->2
    }
    if (c == 0 && sig == 0) {
#pragma unroll
        for (int t = 0; t < T; ++t) red[wave][t][rho] = acc[t];
    }
    __syncthreads();
    const int rows_wg = rgs * RPW;
    for (int i = threadIdx.x; i < rows_wg * T; i += blockDim.x) {
        const int t = i / rows_wg, rl = i - t * rows_wg;
        const int rg = rl / RPW, r = rl - rg * RPW;
        const int64_t rr = (int64_t)blockIdx.x * rows_wg + rl;
        if (rr < n) {
            // the kw partial sums in wave order, whatever the group count
            float v = 0.0f;
            for (int kk = 0; kk < kw; ++kk) v += red[rg * kw + kk][t][r];
            y[t * n + rr] = v;
        }
    }
}

struct GemvArgs {
    const uint8_t *w;
    int64_t n;
    int nsb;
    const int8_t *xq;
    const float *xs;
    const int16_t *xbs;
    float *y;
    int32_t *P, *M;
    int per_wave, kw;
    const float *x;  // fused: f32 activations, and the optional image out
    int8_t *oq;
    float *os;
    int16_t *obs;
};

// A batch of 1-2 stages its image (plus the f32 scales, which the fused
// form keeps beside it) while it fits one workgroup's LDS with room to spare
// (k up to about 128k at batch 1); longer rows read the codes from L2.
constexpr size_t STAGE_MAX = (size_t)144 << 10;

// rows of at most this many superblocks take 16-row steps in the fused GEMV
constexpr int64_t FUSED_SL1_NSB = 16;

static bool staged_image(int64_t t, int64_t k)
{
    return (size_t)t * k * 9 / 8 + (size_t)t * (k / QK) * sizeof(float) <= STAGE_MAX;
}

template <int FMT, int T, int SL, bool PART>
static void launch_one(bool staged, dim3 g, dim3 b, hipStream_t st, const GemvArgs &a)
{
    // staged Q8_K image (codes + bsums), plus the scales when fused
    const size_t img = (size_t)T * a.nsb * QK * 9 / 8;
    if (staged) {
        if constexpr (!PART) {
            if (a.x) {
                hipLaunchKernelGGL((gemv_kernel<FMT, T, SL, false, true, true, 2>), g, b,
                                   img + (size_t)T * a.nsb * sizeof(float), st, a.w, a.n, a.nsb, a.xq, a.xs, a.xbs,
                                   a.y, a.P, a.M, a.per_wave, a.kw, a.x, a.oq, a.os, a.obs);
                return;
            }
        }
        // image chunks (codes, then bsums) per thread of the workgroup; held
        // six at a time before the weight loads where two would not cover
        // them (measured on the dense 17408 x 5120 set: 0.52 -> 0.56 of
        // 8 TB/s; on the FFN matrices six would only cost occupancy)
        const int64_t nst = (int64_t)T * a.nsb * QK / 16 + (int64_t)T * a.nsb * QK / 128;
        if (!PART && nst > 2 * (int64_t)b.x) {
            hipLaunchKernelGGL((gemv_kernel<FMT, T, SL, false, false, true, 6>), g, b, img, st, a.w, a.n, a.nsb, a.xq,
                               a.xs, a.xbs, a.y, a.P, a.M, a.per_wave, a.kw, a.x, a.oq, a.os, a.obs);
            return;
        }
        hipLaunchKernelGGL((gemv_kernel<FMT, T, SL, PART, false, true, 2>), g, b, img, st, a.w, a.n, a.nsb, a.xq,
                           a.xs, a.xbs, a.y, a.P, a.M, a.per_wave, a.kw, a.x, a.oq, a.os, a.obs);
        return;
    }
    hipLaunchKernelGGL((gemv_kernel<FMT, T, SL, PART, false, false, 2>), g, b, 0, st, a.w, a.n, a.nsb, a.xq, a.xs,
                       a.xbs, a.y, a.P, a.M, a.per_wave, a.kw, a.x, a.oq, a.os, a.obs);
}

template <int FMT, int T>
static void launch_sl(bool stg, int sl, bool part, dim3 g, dim3 b, hipStream_t st, const GemvArgs &a)
{
    if (sl == 4) {
        if (part) return launch_one<FMT, T, 4, true>(stg, g, b, st, a);
        return launch_one<FMT, T, 4, false>(stg, g, b, st, a);
    }
    if (part) return launch_one<FMT, T, 1, true>(stg, g, b, st, a);
    return launch_one<FMT, T, 1, false>(stg, g, b, st, a);
}

template <int FMT>
static void launch_t(int t, bool stg, int sl, bool part, dim3 g, dim3 b, hipStream_t st, const GemvArgs &a)
{
    if (t == 1) return launch_sl<FMT, 1>(stg, sl, part, g, b, st, a);
    return launch_sl<FMT, 2>(stg, sl, part, g, b, st, a);
}

static int launch_gemv_one(int fmt, const void *w, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                           const int16_t *xbs, int64_t t, float *y, int32_t *P, int32_t *M, hipStream_t st,
                           const float *x, int8_t *oq, float *os, int16_t *obs)
{
    const int64_t nsb = k / QK;
    // the image is staged in LDS (always, for the fused kernel)
    const bool staged = staged_image(t, k);
    const bool fused = x != nullptr && P == nullptr;
    if (x != nullptr && !fused) return KQ_EINVAL;
    if (fused && !staged) return KQ_EINVAL;  // the fused kernel needs its image in LDS
    // 4 rows x 4 adjacent superblocks per wave step whenever the image is
    // staged in LDS, except in the fused kernel on rows of at most
    // FUSED_SL1_NSB superblocks, which takes 16 rows x one superblock (fewer
    // workgroups, so fewer repeats of the quantisation; measured on the
    // Qwen3-4B W_up matrices at batch 1: 6.18 / 6.95 / 7.04 -> 4.79 / 6.23 /
    // 6.44 us, while the plain GEMV and the longer W_down rows keep 4 x 4).
    // There the fused y sums each row's superblock folds in another order
    // than quantise-then-GEMV, so it matches that within rounding, not bit
    // for bit.  Codes read from L2 take 16 rows x one superblock when that
    // gives two or more workgroups per CU, so that the wave's 16 rows share
    // one superblock's codes.  The choice depends on t, k and n only, so the
    // partials entry point sums in the same order as kq_gemv.
    const int sl = staged ? (fused && nsb <= FUSED_SL1_NSB ? 1 : 4) : ((n + 15) / 16 >= 512 ? 1 : 4);
    const int64_t groups = (n + 16 / sl - 1) / (16 / sl);
    const int64_t nsteps = (nsb + sl - 1) / sl;
    // about 16 waves per CU in flight, at most 16 waves per workgroup, and
    // every wave of a workgroup with the same share of steps; a row of at
    // most 4 steps gives each wave one step (measured: W_up 9728 x 2560 at
    // batch 1, 3 steps, runs 0.2-0.4 us faster with 3 waves of one step than
    // with 2 of up to two, while W_down's 10 steps prefer two per wave).
    int64_t nw = nsteps <= 4 ? nsteps : (4096 + groups - 1) / groups;
    nw = nw < 1 ? 1 : (nw > 16 ? 16 : nw);
    nw = nw > nsteps ? nsteps : nw;
    const int64_t per_wave = (nsteps + nw - 1) / nw;
    const int64_t kw = (nsteps + per_wave - 1) / per_wave;
    // Row groups per workgroup.  Staging a read-only image costs a workgroup
    // little, so the plain GEMV keeps one group per workgroup (the finest
    // grain; grouping it measured slower on W_up, 5.1 -> 6.1 us).  The fused
    // GEMV quantises the whole activation in every workgroup, so it takes
    // as many row groups as 16 waves hold: the fewest workgroups.  Measured
    // on the six FFN matrices at batch 1 (quantise + GEMV in one kernel, sum
    // of the six): 58.4 us at about two workgroups per CU, 53.5-57.9 us at
    // 6-12 waves per workgroup, 42.3 us at 15-16.  Each row's sum order
    // depends only on kw and per_wave, so y does not change with the
    // grouping.
    int64_t rgs = fused ? 16 / kw : 1;
    rgs = rgs > groups ? groups : rgs;
    GemvArgs a{(const uint8_t *)w, n, (int)nsb, xq, xs, xbs, y, P, M, (int)per_wave, (int)kw, x, oq, os, obs};
    const dim3 g((unsigned)((groups + rgs - 1) / rgs)), b((unsigned)(64 * kw * rgs));
    const bool part = P != nullptr;
    if (fmt == KQ_Q4_K) launch_t<KQ_Q4_K>((int)t, staged, sl, part, g, b, st, a);
    else if (fmt == KQ_Q5_K) launch_t<KQ_Q5_K>((int)t, staged, sl, part, g, b, st, a);
    else launch_t<KQ_Q6_K>((int)t, staged, sl, part, g, b, st, a);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ELAUNCH;
}

// Whether the one-kernel quantise + GEMV (launch_gemv with x) takes t x k:
// a batch of 1-2 whose image and scales fit the LDS stage.
bool gemv_fusable(int64_t t, int64_t k) { return t <= 2 && staged_image(t, k); }

int launch_gemv_mma(int fmt, const void *w, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                    const int16_t *xbs, int64_t t, float *y, int32_t *P, int32_t *M, hipStream_t st);

// Batches 1-2 on the dot-product GEMV above (the fused form included);
// batches 3-8 on the matrix cores, whose work per weight byte does not grow
// with the batch.  The choice depends on t only, so the partials entry
// point takes the same kernel.
int launch_gemv(int fmt, const void *w, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                const int16_t *xbs, int64_t t, float *y, int32_t *P, int32_t *M, hipStream_t st,
                const float *x, int8_t *oq, float *os, int16_t *obs)
{
    if (t >= 3) {
        if (x != nullptr) return KQ_EINVAL;  // the fused form is batches 1-2
        return launch_gemv_mma(fmt, w, n, k, xq, xs, xbs, t, y, P, M, st);
    }
    return launch_gemv_one(fmt, w, n, k, xq, xs, xbs, t, y, P, M, st, x, oq, os, obs);
}

}  // namespace kq
