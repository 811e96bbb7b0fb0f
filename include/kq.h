/*
 * kq.h -- C ABI of the K-quant weight x Q8_K activation matmul ("kq v2")
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (K-quant kernel arc page, daScript PR "dasLLAMA: K-quant
 * kernel arc -- kq v2 integer folds, kq v3 panel-scratch tiles, chain
 * regrain, parity gates"; section "The pieces", kq v2 item, and the k4 v2
 * and k5/k6 v2 commit messages):
 *
 *   y[t][n] = sum over superblocks s of ONE float fold of integer partials
 *     Q4_K, Q5_K:  d*d8*P - dmin*d8*M
 *                  P = sum_j sc_j * (sum over sub-block j of q_i * a_i)
 *                  M = sum_j m_j * (bsum_{2j} + bsum_{2j+1})
 *     Q6_K:        d*d8*(iacc - 32*bacc)
 *                  iacc = sum_j sc_j * (sum over 16-wide sub-block j of q_i * a_i)
 *                  bacc = sum_j sc_j * bsum_j
 *
 * where the weight row n is a sequence of 256-weight ggml superblocks
 * (Q4_K 144 B, Q5_K 176 B, Q6_K 210 B records) and the activation row t is
 * in Q8_K form: a[k] int8, one float scale d8 per 256 and an int16 sum per
 * 16 (bsum).  Q5_K shares Q4_K's 6-bit scale/min block and adds a fifth
 * quant bit; Q6_K carries signed 8-bit scales per 16 weights.  The
 * activation is always quantised to Q8_K before the dot (the k5/k6 v2
 * commit message: the matmuls always quantize Q8_K), and K must cover
 * whole superblocks (the chain-regrain commit message: dim % 256 for any
 * kq weight).
 *
 * Conventions shared by every entry point:
 *  - Buffers.  Every pointer argument except the host side of a copy is a
 *    DEVICE pointer on the current HIP device, owned by the caller.  The
 *    library allocates nothing.  Its only global state is on the host: the
 *    CU count, read once, and an atomic call counter that tags the GEMM's
 *    split counters; calls are reentrant and thread-safe.
 *  - Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream).  Every call only enqueues work and returns; nothing
 *    synchronises.  Outputs are fully overwritten.
 *  - Layouts.  Row-major and dense: x[t][k], xq[t][k], xs[t][k/256],
 *    xbs[t][k/16], y[t][n], partials[t][n][k/256] -- except the codes and
 *    bsums that kq_gemm_tiles and kq_gemm_grouped read, which come in the
 *    tile image (kq_quantize_q8k_tiles).
 *  - Alignment.  w_ggml, w_planes, x, xq and xbs must be 16-byte aligned;
 *    xs, y and the partials 4-byte aligned.
 *  - Errors.  All arguments are checked on the host before any HIP call, so
 *    a bad call returns its code without touching the device.  A failed
 *    kernel launch returns KQ_ELAUNCH.  No exceptions cross the ABI.
 */
#ifndef KQ_H
#define KQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* the library is built with hidden visibility: only these entry points are
 * exported */
#if defined(__GNUC__) || defined(__clang__)
#pragma GCC visibility push(default)
#endif

/* Weight formats (the ggml K-quant records). */
typedef enum { KQ_Q4_K = 4, KQ_Q5_K = 5, KQ_Q6_K = 6 } kq_format;

/* Status codes. */
enum {
    KQ_OK = 0,
    KQ_EINVAL = -1,  /* a size is out of range, or a pointer is NULL */
    KQ_EFORMAT = -2, /* unknown weight format */
    KQ_EALIGN = -3,  /* a pointer is not aligned as required */
    KQ_ELAUNCH = -4  /* the HIP launch failed */
};

/* Bytes of one ggml superblock record of `fmt` (144, 176, 210), or 0. */
size_t kq_record_bytes(int fmt);

/* Bytes of the device planes that kq_pack writes for an n x k matrix of
 * `fmt`, or 0 on bad arguments (n < 1, k < 256, k % 256 != 0, bad fmt).
 * It is the ggml byte count plus at most 255 bytes of alignment padding
 * per plane. */
size_t kq_packed_bytes(int fmt, int64_t n, int64_t k);

/* Re-lay ggml superblock records w_ggml[n][k/256] (record bytes as on
 * disk) into the device planes w_planes (kq_packed_bytes bytes).  The
 * planes hold every byte of the records, split by field (K-quant kernel
 * arc page, "The pieces", kq v3 item: the DRAM planes keep the packed
 * 144/176/210 B per superblock), so the matmul's loads are 16-byte
 * aligned and coalesced.  One-time, at load. */
int kq_pack(int fmt, const void *w_ggml, int64_t n, int64_t k, void *w_planes, void *stream);

/* Inverse of kq_pack: planes back to ggml records (for round-trip tests). */
int kq_unpack(int fmt, const void *w_planes, int64_t n, int64_t k, void *w_ggml, void *stream);

/* Q8_K quantisation of float activations x[t][k]: per 256 values
 * amax = max|x|, d8 = amax/127 (IEEE binary32 division), a = rint(x/d8)
 * (binary32 division, round half to even), clamped to [-127, 127]; an
 * all-zero chunk gives d8 = 0 and a = 0; xbs holds the sum of each 16
 * codes (K-quant kernel arc page, "The pieces", kq v2 item; the k4 v2
 * commit message).  Outputs xq[t][k] int8, xs[t][k/256] float,
 * xbs[t][k/16] int16.  t >= 1.  x must be finite. */
int kq_quantize_q8k(const float *x, int64_t t, int64_t k, int8_t *xq, float *xs, int16_t *xbs,
                    void *stream);

/* Bytes of the codes of the tile image of t tokens of k: t rounded up to a
 * multiple of 32, times k; 0 on bad arguments.  Its bsums take 1/8 of that. */
size_t kq_q8k_tiles_bytes(int64_t t, int64_t k);

/* kq_quantize_q8k writing the tile image the GEMM reads: the same Q8_K
 * values (xs row-major and bit-identical), with the codes and bsums laid out
 * as the operands of the int8 and f16 32x32 MFMAs.  Tokens in groups of 32:
 *   codes, kq_q8k_tiles_bytes(t, k) bytes: for group g and 32-code K chunk
 *     c a 1 KiB block; byte ((q*32 + r)*16 + e), q in 0..1, r in 0..31, e
 *     in 0..15, is code 32c + 16q + e of token 32g + r:
 *     xq_tiles[((g*(k/32) + c)*64 + q*32 + r)*16 + e] = xq[32g + r][32c + 16q + e];
 *   bsums, IEEE binary16 (exact: |bsum| <= 2032), kq_q8k_tiles_bytes/8
 *     bytes: for group g and superblock s a 1 KiB block;
 *     xbs_tiles[((g*(k/256) + s)*64 + q*32 + r)*8 + e] = xbs[32g + r][16s + 8q + e].
 * Each MFMA operand is then one coalesced 1 KiB load.  Tokens t .. (rounded
 * up to 32) - 1 get zero codes and zero bsums. */
int kq_quantize_q8k_tiles(const float *x, int64_t t, int64_t k, int8_t *xq_tiles, float *xs, uint16_t *xbs_tiles,
                          void *stream);

/* kq_quantize_q8k_tiles of gathered rows, for the grouped GEMM: image row
 * i (0 <= i < m) is the Q8_K of activation row rows[i] of x[t][k]; an index
 * outside [0, t) gives a zero row (codes 0, bsums 0, d8 = 0).  rows is a
 * device int32[m]; xs has m rows; the tile buffers hold m rounded up to 32
 * rows (kq_q8k_tiles_bytes(m, k)).  A mixture-of-experts layer lists the
 * tokens routed to each expert one expert after another, each expert's
 * list padded with -1 to a multiple of 32 rows (K-quant kernel arc page,
 * "The pieces", kq v2 item: the MoE path fills one Q8_K image for gate and
 * up). */
int kq_quantize_q8k_tiles_gather(const float *x, int64_t t, int64_t k, const int32_t *rows, int64_t m,
                                 int8_t *xq_tiles, float *xs, uint16_t *xbs_tiles, void *stream);

/* Decode GEMV, batch t in 1..8: y[t][n] = W . a_t by the folds above,
 * streaming the packed planes once. */
int kq_gemv(int fmt, const void *w_planes, int64_t n, int64_t k, const int8_t *xq, const float *xs,
            const int16_t *xbs, int64_t t, float *y, void *stream);

/* Decode GEMV with the Q8_K quantisation fused in: f32 activations
 * x[t][k], t in 1..8, in; y[t][n] out.  The quantisation is the one of
 * kq_quantize_q8k, bit for bit; the kernel-arc page's chain regrain
 * (commit message of that name) quantises inside the consuming chain at
 * whole-superblock granules -- here inside the GEMV, which saves the
 * separate quantiser launch and the image's round trip.  For t <= 2 this
 * is one kernel while the image and its scales fit one workgroup's LDS
 * stage (t*k*9/8 + t*(k/256)*4 <= 147456 bytes: k up to 129024 at t = 1,
 * 64512 at t = 2):
 * every workgroup quantises x into LDS (a workgroup covers as many row
 * groups as 16 waves hold, so few of them repeat it); xq/xs/xbs may then
 * be NULL (all three), or receive the Q8_K image.  Past that size, and for
 * t > 2, the image buffers are required (KQ_EINVAL without them) and the
 * call runs kq_quantize_q8k then kq_gemv.  The image and every
 * superblock's fold are those of kq_quantize_q8k then kq_gemv, and so is y,
 * bit for bit, except in the one-kernel form on rows of at most 16
 * superblocks (k <= 4096), whose steps cover 16 rows x one superblock: there
 * each row sums its superblock folds in another order, and y matches
 * quantise-then-GEMV within float rounding.
 * x must be 16-byte aligned and finite. */
int kq_gemv_f32(int fmt, const void *w_planes, int64_t n, int64_t k, const float *x, int64_t t,
                float *y, int8_t *xq, float *xs, int16_t *xbs, void *stream);

/* Bytes of the workspace kq_gemm and kq_gemm_partials need for this shape on
 * the current device, or 0 on bad arguments (see kq_gemm). */
size_t kq_gemm_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t m);

/* Prefill GEMM, m >= 1 tokens: y[m][n], the folds of kq_gemv, from the Q8_K
 * row image that kq_quantize_q8k writes (xq[m][k], xs[m][k/256],
 * xbs[m][k/16] int16) -- the pages' matmul sequence: quantise to Q8_K, then
 * dot (K-quant kernel arc page, k5/k6 v2 commit message; the regrain commit
 * message keeps one activation image per consumed form).
 * workspace: a 256-byte aligned device buffer of workspace_bytes >=
 * kq_gemm_workspace_bytes(fmt, n, k, m) bytes (no initial contents needed;
 * KQ_EINVAL if NULL or smaller).  The call first re-lays the image into the
 * tile form at the start of the workspace (kq_quantize_q8k_tiles's layout,
 * bit for bit), then runs kq_gemm_tiles on it with the rest of the workspace
 * as that call's k-split workspace, so y is bit-identical to
 * kq_quantize_q8k_tiles + kq_gemm_tiles with the same split.  Calls sharing
 * one workspace must be ordered on one stream.  k <= 2^23 - 256. */
int kq_gemm(int fmt, const void *w_planes, int64_t n, int64_t k, const int8_t *xq, const float *xs,
            const int16_t *xbs, int64_t m, float *y, void *workspace, size_t workspace_bytes, void *stream);

/* Size of the device array kq_gemm_noalloc uses as its workspace. */
#define KQ_SCRATCH_BYTES ((size_t)64 << 20)

/* kq_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same call without the workspace argument.  Its workspace is a file-scope
 * device array of KQ_SCRATCH_BYTES (64 MiB) inside the library, one per
 * GPU, held until the process ends; each device's address is looked up on
 * the first call on that device.  The call allocates nothing, and y is
 * bit-identical to kq_gemm's.  KQ_EINVAL if kq_gemm_workspace_bytes(fmt, n,
 * k, m) exceeds KQ_SCRATCH_BYTES (e.g. m * k above about 5.9e7 with no
 * k split).  Every call on one GPU shares that GPU's array and leaves its
 * contents behind (nothing in it needs clearing: the re-laid image is
 * rewritten by every call, and the k-split counters are tagged per call), so
 * calls that overlap on one GPU -- on different streams, or from different
 * threads without ordering -- race and must not be issued. */
int kq_gemm_noalloc(int fmt, const void *w_planes, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                    const int16_t *xbs, int64_t m, float *y, void *stream);

/* Bytes of the optional kq_gemm_tiles workspace for this shape on the current
 * device (0: kq_gemm_tiles would not use one), or 0 on bad arguments. */
size_t kq_gemm_tiles_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t m);

/* Token count of the tile kq_gemm / kq_gemm_tiles runs for this shape: 32
 * (the 32-token tile, whose tiles pair up on 64-row panels where their count
 * allows) or 256 (the 256-token tile); 0 on bad arguments. */
int kq_gemm_tile_tokens(int fmt, int64_t n, int64_t k, int64_t m);

/* Prefill GEMM, m >= 1 tokens, on the tile image of kq_quantize_q8k_tiles
 * (codes and f16 bsums in MFMA operand order, xs row-major): y[m][n], the
 * folds of kq_gemv.  k <= 2^23 - 256 (KQ_EINVAL above).  m <= 192 runs a
 * 32-token tile that unpacks each weight once per 32 tokens, or per 64 when
 * the tiles pair up (33..64 and 97..192 tokens; with a workspace, Q4_K/Q5_K
 * also pair 65..96 tokens and split tiles of up to 32, the last pair's
 * second tile empty; in registers for Q6_K, through an LDS panel for
 * Q4_K/Q5_K); m >= 193 a 256-token tile that unpacks it once per 256 tokens
 * into LDS.
 * workspace: NULL, or a 256-byte aligned device buffer of workspace_bytes >=
 * kq_gemm_tiles_workspace_bytes bytes (no initial contents needed; a
 * non-NULL pointer where that size is 0).  With it, a grid too small to fill
 * the GPU is split along k: for the 256-token tile each tile's parts write
 * partial sums to the workspace and the last part of the tile to finish adds
 * them into y (one launch); for the 32-token tile the waves of a workgroup
 * take two to four parts of k and add them in LDS where the grid still runs
 * in one round, and whole-output slices that a second kernel adds take the
 * rest.  All add in split order, so results are the same from call to call
 * (they may differ from the unsplit sum in the last bits, within the fold's
 * float tolerance).  The
 * 256-token tile's parts count in through counter words at the start of the
 * workspace that every call tags as its own, so stale contents are ignored
 * and graph replays may reuse the workspace.  Calls sharing one workspace
 * must be ordered on one stream.  A NULL or too small workspace runs
 * unsplit. */
int kq_gemm_tiles(int fmt, const void *w_planes, int64_t n, int64_t k, const int8_t *xq_tiles, const float *xs,
                  const uint16_t *xbs_tiles, int64_t m, float *y, void *workspace, size_t workspace_bytes,
                  void *stream);

/* kq_gemv that also stores each superblock's int32 partials:
 * P[t][n][k/256] and M[t][n][k/256] (Q6_K: P = iacc - 32*bacc and M = 0;
 * M may be NULL for Q6_K).  The same kernel body as kq_gemv. */
int kq_gemv_partials(int fmt, const void *w_planes, int64_t n, int64_t k, const int8_t *xq,
                     const float *xs, const int16_t *xbs, int64_t t, float *y, int32_t *P,
                     int32_t *M, void *stream);

/* Grouped GEMM of a mixture-of-experts layer, all experts in one launch:
 * `experts` weight matrices of n x k in one format, expert e's planes at
 * w_planes + e * w_stride bytes (w_stride >= kq_packed_bytes(fmt, n, k), a
 * multiple of 16); a tile image of m rows (kq_quantize_q8k_tiles_gather)
 * whose 32-row tile i belongs to expert tile_expert[i] (device
 * int32[ceil(m/32)]).  y[m][n]: row i is row i of the image times that
 * expert's matrix.  A tile whose expert id is outside [0, experts) is left
 * unwritten.  Unsplit; each tile runs the kq_gemm_tiles 32-token tile body, so a
 * tile's outputs equal kq_gemm_tiles's on the same rows bit for bit. */
int kq_gemm_grouped(int fmt, const void *w_planes, int64_t w_stride, int64_t experts, const int32_t *tile_expert,
                    int64_t n, int64_t k, const int8_t *xq_tiles, const float *xs, const uint16_t *xbs_tiles,
                    int64_t m, float *y, void *stream);

/* kq_gemm (unsplit) that also stores the int32 partials, as
 * kq_gemv_partials; same row image and workspace as kq_gemm. */
int kq_gemm_partials(int fmt, const void *w_planes, int64_t n, int64_t k, const int8_t *xq, const float *xs,
                     const int16_t *xbs, int64_t m, float *y, int32_t *P, int32_t *M, void *workspace,
                     size_t workspace_bytes, void *stream);

/* kq_gemm_tiles (unsplit, no workspace) that also stores the int32
 * partials, as kq_gemv_partials. */
int kq_gemm_tiles_partials(int fmt, const void *w_planes, int64_t n, int64_t k, const int8_t *xq_tiles,
                           const float *xs, const uint16_t *xbs_tiles, int64_t m, float *y, int32_t *P,
                           int32_t *M, void *stream);

/* Static text for a status code. */
const char *kq_strerror(int code);

#if defined(__GNUC__) || defined(__clang__)
#pragma GCC visibility pop
#endif

#ifdef __cplusplus
}
#endif

#endif /* KQ_H */
