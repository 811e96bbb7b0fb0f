// kq_api.hip -- the C ABI declared in include/kq.h: argument checks on the
// host (before any HIP call, so a bad call never touches the device), then
// the launch on the caller's stream.
#include <limits.h>

#include <atomic>

#include "kq_common.h"

namespace kq {
int launch_quantize_q8k(const float *x, int64_t t, int64_t k, int8_t *xq, float *xs, int16_t *xbs,
                        hipStream_t stream);
int launch_quantize_q8k_tiles(const float *x, int64_t t, int64_t k, int8_t *xq, float *xs, int16_t *xbs,
                              hipStream_t stream);
int launch_relay_tiles(const int8_t *xq, const int16_t *xbs, int64_t m, int64_t k, int8_t *xqt, uint16_t *xbt,
                       hipStream_t stream);
int launch_quantize_q8k_tiles_gather(const float *x, int64_t t, const int32_t *src, int64_t m, int64_t k,
                                     int8_t *xq, float *xs, int16_t *xbs, hipStream_t stream);
int launch_gemm_mid(int fmt, const void *w, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                    const void *xbs, int64_t m, float *y, int32_t *P, int32_t *M, void *ws, size_t ws_bytes,
                    hipStream_t st);
size_t gemm_mid_workspace_bytes(int64_t n, int64_t k, int64_t m);
int launch_gemm_grouped(int fmt, const void *w, int64_t w_stride, int64_t experts, const int32_t *tile_expert,
                        int64_t n, int64_t k, const int8_t *xq, const float *xs, const void *xbs, int64_t m,
                        float *y, int32_t *P, int32_t *M, hipStream_t st);
// token counts up to GEMM_MID_MAX run the 32-token tile (above 127 tokens
// its tiles pair up and beat a 256-token tile that would run at most
// three-quarters full); the rest run the 256-token prefill tile
constexpr int64_t GEMM_MID_MAX = 192;
inline bool gemm_uses_mid(int64_t m) { return m <= GEMM_MID_MAX; }
int launch_pack(int fmt, const void *w_ggml, int64_t n, int64_t k, void *w_planes, hipStream_t stream);
int launch_unpack(int fmt, const void *w_planes, int64_t n, int64_t k, void *w_ggml, hipStream_t stream);
bool gemv_fusable(int64_t t, int64_t k);
int launch_gemv(int fmt, const void *w, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                const int16_t *xbs, int64_t t, float *y, int32_t *P, int32_t *M, hipStream_t st,
                const float *x = nullptr, int8_t *oq = nullptr, float *os = nullptr, int16_t *obs = nullptr);
int launch_gemm(int fmt, const void *w, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                const void *xbs, int64_t m, float *y, int32_t *P, int32_t *M, void *ws, size_t ws_bytes,
                hipStream_t st);
size_t gemm_workspace_bytes(int64_t n, int64_t k, int64_t m);
}  // namespace kq

namespace {

bool known(int fmt) { return fmt == KQ_Q4_K || fmt == KQ_Q5_K || fmt == KQ_Q6_K; }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// n x k weight matrix: n >= 1, k a positive multiple of 256, both < 2^31
int check_nk(int64_t n, int64_t k)
{
    if (n < 1 || n > INT_MAX || k < kq::QK || k > INT_MAX || k % kq::QK) return KQ_EINVAL;
    return KQ_OK;
}

// operands of one matmul call
int check_matmul(int fmt, const void *w, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                 const int16_t *xbs, int64_t t, int64_t tmax, const float *y, const int32_t *P,
                 const int32_t *M, bool partials)
{
    if (!known(fmt)) return KQ_EFORMAT;
    if (check_nk(n, k)) return KQ_EINVAL;
    if (t < 1 || t > tmax) return KQ_EINVAL;
    // the grid and every row-major offset stay inside int64 / uint32
    if (n * t > ((int64_t)1 << 40)) return KQ_EINVAL;
    // the GEMM addresses 256 tokens of codes with 32-bit offsets
    if (tmax > 8 && k > kq::GEMM_KMAX) return KQ_EINVAL;
    if (!w || !xq || !xs || !xbs || !y) return KQ_EINVAL;
    if (partials && (!P || (fmt != KQ_Q6_K && !M))) return KQ_EINVAL;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(xbs, 16) || !aligned(xs, 4) || !aligned(y, 4))
        return KQ_EALIGN;
    if (partials && (!aligned(P, 4) || (M && !aligned(M, 4)))) return KQ_EALIGN;
    return KQ_OK;
}

// t rows of k activations: the quantiser's grid (4 chunks per workgroup,
// rows rounded up to 16) must fit gridDim.x < 2^31
int check_quantize(const float *x, int64_t t, int64_t k, const int8_t *xq, const float *xs, const int16_t *xbs)
{
    if (t < 1 || t > INT_MAX || check_nk(1, k) || !x || !xq || !xs || !xbs) return KQ_EINVAL;
    if ((t + 15) * (k / kq::QK) > ((int64_t)1 << 32)) return KQ_EINVAL;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(xbs, 16) || !aligned(xs, 4)) return KQ_EALIGN;
    return KQ_OK;
}

}  // namespace

extern "C" {

size_t kq_record_bytes(int fmt) { return known(fmt) ? (size_t)kq::record_bytes(fmt) : 0; }

size_t kq_packed_bytes(int fmt, int64_t n, int64_t k)
{
    if (!known(fmt) || check_nk(n, k)) return 0;
    return (size_t)kq::planes_of(fmt, n, k / kq::QK).total;
}

int kq_pack(int fmt, const void *w_ggml, int64_t n, int64_t k, void *w_planes, void *stream)
{
    if (!known(fmt)) return KQ_EFORMAT;
    if (check_nk(n, k) || !w_ggml || !w_planes) return KQ_EINVAL;
    if (!aligned(w_ggml, 16) || !aligned(w_planes, 16)) return KQ_EALIGN;
    return kq::launch_pack(fmt, w_ggml, n, k, w_planes, (hipStream_t)stream);
}

int kq_unpack(int fmt, const void *w_planes, int64_t n, int64_t k, void *w_ggml, void *stream)
{
    if (!known(fmt)) return KQ_EFORMAT;
    if (check_nk(n, k) || !w_ggml || !w_planes) return KQ_EINVAL;
    if (!aligned(w_ggml, 16) || !aligned(w_planes, 16)) return KQ_EALIGN;
    return kq::launch_unpack(fmt, w_planes, n, k, w_ggml, (hipStream_t)stream);
}

int kq_quantize_q8k(const float *x, int64_t t, int64_t k, int8_t *xq, float *xs, int16_t *xbs, void *stream)
{
    int rc = check_quantize(x, t, k, xq, xs, xbs);
    if (rc) return rc;
    return kq::launch_quantize_q8k(x, t, k, xq, xs, xbs, (hipStream_t)stream);
}

size_t kq_q8k_tiles_bytes(int64_t t, int64_t k)
{
    if (t < 1 || t > INT_MAX || check_nk(1, k)) return 0;
    return (size_t)((t + 31) / 32 * 32) * (size_t)k;
}

int kq_quantize_q8k_tiles(const float *x, int64_t t, int64_t k, int8_t *xq_tiles, float *xs, uint16_t *xbs_tiles,
                          void *stream)
{
    int rc = check_quantize(x, t, k, xq_tiles, xs, (const int16_t *)xbs_tiles);
    if (rc) return rc;
    return kq::launch_quantize_q8k_tiles(x, t, k, xq_tiles, xs, (int16_t *)xbs_tiles, (hipStream_t)stream);
}

int kq_quantize_q8k_tiles_gather(const float *x, int64_t t, int64_t k, const int32_t *rows, int64_t m,
                                 int8_t *xq_tiles, float *xs, uint16_t *xbs_tiles, void *stream)
{
    int rc = check_quantize(x, t, k, xq_tiles, xs, (const int16_t *)xbs_tiles);
    if (rc) return rc;
    if (!rows || m < 1 || m > INT_MAX || (m + 31) * (k / kq::QK) > ((int64_t)1 << 32)) return KQ_EINVAL;
    if (!aligned(rows, 4)) return KQ_EALIGN;
    return kq::launch_quantize_q8k_tiles_gather(x, t, rows, m, k, xq_tiles, xs, (int16_t *)xbs_tiles,
                                                (hipStream_t)stream);
}

int kq_gemv(int fmt, const void *w_planes, int64_t n, int64_t k, const int8_t *xq, const float *xs,
            const int16_t *xbs, int64_t t, float *y, void *stream)
{
    int rc = check_matmul(fmt, w_planes, n, k, xq, xs, xbs, t, 8, y, nullptr, nullptr, false);
    if (rc) return rc;
    return kq::launch_gemv(fmt, w_planes, n, k, xq, xs, xbs, t, y, nullptr, nullptr, (hipStream_t)stream);
}

int kq_gemv_f32(int fmt, const void *w_planes, int64_t n, int64_t k, const float *x, int64_t t, float *y,
                int8_t *xq, float *xs, int16_t *xbs, void *stream)
{
    if (!known(fmt)) return KQ_EFORMAT;
    if (check_nk(n, k) || t < 1 || t > 8 || !w_planes || !x || !y) return KQ_EINVAL;
    const bool image = xq || xs || xbs;
    if (image && !(xq && xs && xbs)) return KQ_EINVAL;  // all three or none
    if (t > 2 && !image) return KQ_EINVAL;              // batches past 2 need the image buffers
    if (!aligned(w_planes, 16) || !aligned(x, 16) || !aligned(y, 4)) return KQ_EALIGN;
    if (image && (!aligned(xq, 16) || !aligned(xbs, 16) || !aligned(xs, 4))) return KQ_EALIGN;
    // Batches of 1-2 run as one kernel (each workgroup quantises x into its
    // LDS stage) while the image fits that stage; the image buffers, when
    // given, then receive the image too.  Otherwise the quantiser and the
    // GEMV run as two launches, which needs the buffers.  y is the same bits
    // either way.
    if (kq::gemv_fusable(t, k))
        return kq::launch_gemv(fmt, w_planes, n, k, nullptr, nullptr, nullptr, t, y, nullptr, nullptr,
                               (hipStream_t)stream, x, xq, xs, xbs);
    if (!image) return KQ_EINVAL;
    int rc = kq::launch_quantize_q8k(x, t, k, xq, xs, xbs, (hipStream_t)stream);
    if (rc) return rc;
    return kq::launch_gemv(fmt, w_planes, n, k, xq, xs, xbs, t, y, nullptr, nullptr, (hipStream_t)stream);
}

int kq_gemv_partials(int fmt, const void *w_planes, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                     const int16_t *xbs, int64_t t, float *y, int32_t *P, int32_t *M, void *stream)
{
    int rc = check_matmul(fmt, w_planes, n, k, xq, xs, xbs, t, 8, y, P, M, true);
    if (rc) return rc;
    return kq::launch_gemv(fmt, w_planes, n, k, xq, xs, xbs, t, y, P, M, (hipStream_t)stream);
}

size_t kq_gemm_tiles_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t m)
{
    if (!known(fmt) || check_nk(n, k) || m < 1 || m > INT_MAX || k > kq::GEMM_KMAX) return 0;
    return kq::gemm_uses_mid(m) ? kq::gemm_mid_workspace_bytes(n, k, m) : kq::gemm_workspace_bytes(n, k, m);
}

int kq_gemm_tile_tokens(int fmt, int64_t n, int64_t k, int64_t m)
{
    if (!known(fmt) || check_nk(n, k) || m < 1 || m > INT_MAX || k > kq::GEMM_KMAX) return 0;
    return kq::gemm_uses_mid(m) ? 32 : 256;
}

int kq_gemm_tiles(int fmt, const void *w_planes, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                  const uint16_t *xbs, int64_t m, float *y, void *workspace, size_t workspace_bytes, void *stream)
{
    int rc = check_matmul(fmt, w_planes, n, k, xq, xs, (const int16_t *)xbs, m, INT_MAX, y, nullptr, nullptr,
                          false);
    if (rc) return rc;
    if (workspace && !aligned(workspace, 256)) return KQ_EALIGN;
    if (kq::gemm_uses_mid(m))
        return kq::launch_gemm_mid(fmt, w_planes, n, k, xq, xs, xbs, m, y, nullptr, nullptr, workspace,
                                   workspace_bytes, (hipStream_t)stream);
    return kq::launch_gemm(fmt, w_planes, n, k, xq, xs, xbs, m, y, nullptr, nullptr, workspace, workspace_bytes,
                           (hipStream_t)stream);
}

int kq_gemm_grouped(int fmt, const void *w_planes, int64_t w_stride, int64_t experts, const int32_t *tile_expert,
                    int64_t n, int64_t k, const int8_t *xq_tiles, const float *xs, const uint16_t *xbs_tiles,
                    int64_t m, float *y, void *stream)
{
    int rc = check_matmul(fmt, w_planes, n, k, xq_tiles, xs, (const int16_t *)xbs_tiles, m, INT_MAX, y, nullptr,
                          nullptr, false);
    if (rc) return rc;
    if (!tile_expert || experts < 1 || experts > INT_MAX) return KQ_EINVAL;
    if (w_stride < (int64_t)kq::planes_of(fmt, n, k / kq::QK).total) return KQ_EINVAL;
    if (w_stride % 16 || !aligned(tile_expert, 4)) return KQ_EALIGN;
    return kq::launch_gemm_grouped(fmt, w_planes, w_stride, experts, tile_expert, n, k, xq_tiles, xs, xbs_tiles, m, y,
                                   nullptr, nullptr, (hipStream_t)stream);
}

int kq_gemm_tiles_partials(int fmt, const void *w_planes, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                           const uint16_t *xbs, int64_t m, float *y, int32_t *P, int32_t *M, void *stream)
{
    int rc = check_matmul(fmt, w_planes, n, k, xq, xs, (const int16_t *)xbs, m, INT_MAX, y, P, M, true);
    if (rc) return rc;
    if (kq::gemm_uses_mid(m))
        return kq::launch_gemm_mid(fmt, w_planes, n, k, xq, xs, xbs, m, y, P, M, nullptr, 0, (hipStream_t)stream);
    return kq::launch_gemm(fmt, w_planes, n, k, xq, xs, xbs, m, y, P, M, nullptr, 0, (hipStream_t)stream);
}

// The row-image GEMM's workspace: the tile image of the m tokens (codes, then
// f16 bsums, each 256-byte aligned), then the tile GEMM's k-split workspace.
struct RowWs {
    size_t codes, bsums, split, total;
};

static RowWs row_ws(int fmt, int64_t n, int64_t k, int64_t m)
{
    RowWs w{};
    const size_t tb = kq_q8k_tiles_bytes(m, k);
    if (!tb) return w;
    w.codes = 0;
    w.bsums = (size_t)kq::align256((int64_t)tb);
    w.split = w.bsums + (size_t)kq::align256((int64_t)(tb / 8));
    w.total = w.split + kq_gemm_tiles_workspace_bytes(fmt, n, k, m);
    return w;
}

size_t kq_gemm_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t m)
{
    if (!known(fmt) || check_nk(n, k) || m < 1 || m > INT_MAX || k > kq::GEMM_KMAX) return 0;
    return row_ws(fmt, n, k, m).total;
}

// the row-image calls: re-lay into the workspace, then the tile GEMM
static int gemm_rows(int fmt, const void *w_planes, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                     const int16_t *xbs, int64_t m, float *y, int32_t *P, int32_t *M, void *workspace,
                     size_t workspace_bytes, void *stream)
{
    int rc = check_matmul(fmt, w_planes, n, k, xq, xs, xbs, m, INT_MAX, y, P, M, P != nullptr);
    if (rc) return rc;
    if ((m + 31) * (k / kq::QK) > ((int64_t)1 << 32)) return KQ_EINVAL;
    const RowWs l = row_ws(fmt, n, k, m);
    if (!workspace || workspace_bytes < l.total) return KQ_EINVAL;
    if (!aligned(workspace, 256)) return KQ_EALIGN;
    char *ws = (char *)workspace;
    int8_t *xqt = (int8_t *)(ws + l.codes);
    uint16_t *xbt = (uint16_t *)(ws + l.bsums);
    rc = kq::launch_relay_tiles(xq, xbs, m, k, xqt, xbt, (hipStream_t)stream);
    if (rc) return rc;
    if (P) return kq_gemm_tiles_partials(fmt, w_planes, n, k, xqt, xs, xbt, m, y, P, M, stream);
    return kq_gemm_tiles(fmt, w_planes, n, k, xqt, xs, xbt, m, y, ws + l.split, workspace_bytes - l.split, stream);
}

int kq_gemm(int fmt, const void *w_planes, int64_t n, int64_t k, const int8_t *xq, const float *xs,
            const int16_t *xbs, int64_t m, float *y, void *workspace, size_t workspace_bytes, void *stream)
{
    return gemm_rows(fmt, w_planes, n, k, xq, xs, xbs, m, y, nullptr, nullptr, workspace, workspace_bytes, stream);
}

int kq_gemm_partials(int fmt, const void *w_planes, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                     const int16_t *xbs, int64_t m, float *y, int32_t *P, int32_t *M, void *workspace,
                     size_t workspace_bytes, void *stream)
{
    if (!P) return KQ_EINVAL;
    return gemm_rows(fmt, w_planes, n, k, xq, xs, xbs, m, y, P, M, workspace, workspace_bytes, stream);
}

}  // extern "C"

// The workspace of kq_gemm_noalloc: a file-scope device array, one copy per
// GPU, held until the process ends.  Host code never names it directly (its
// host-side name is not a device address): the entry point looks up each
// device's address once, with that device current, and passes that.
static __device__ __align__(256) uint8_t scratch[KQ_SCRATCH_BYTES];

namespace {
constexpr int SCRATCH_DEVICES = 64;
std::atomic<void *> scratch_ptr[SCRATCH_DEVICES];

// this device's copy of `scratch`, or nullptr if it cannot be found
void *scratch_of_current_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_DEVICES) return nullptr;
    void *p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        // racing first calls on one device look up the same address
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}
}  // namespace

extern "C" {

int kq_gemm_noalloc(int fmt, const void *w_planes, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                    const int16_t *xbs, int64_t m, float *y, void *stream)
{
    int rc = check_matmul(fmt, w_planes, n, k, xq, xs, xbs, m, INT_MAX, y, nullptr, nullptr, false);
    if (rc) return rc;
    const size_t need = kq_gemm_workspace_bytes(fmt, n, k, m);
    if (need == 0 || need > KQ_SCRATCH_BYTES) return KQ_EINVAL;
    void *ws = scratch_of_current_device();
    if (!ws) return KQ_ELAUNCH;
    return gemm_rows(fmt, w_planes, n, k, xq, xs, xbs, m, y, nullptr, nullptr, ws, KQ_SCRATCH_BYTES, stream);
}

const char *kq_strerror(int code)
{
    switch (code) {
    case KQ_OK: return "ok";
    case KQ_EINVAL: return "invalid argument (size out of range or NULL pointer)";
    case KQ_EFORMAT: return "unknown weight format";
    case KQ_EALIGN: return "misaligned pointer";
    case KQ_ELAUNCH: return "HIP kernel launch failed";
    default: return "unknown status code";
    }
}

}  // extern "C"
