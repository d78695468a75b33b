/*
 * nf4.h -- C ABI of libnf4.so: an NF4-style 4-bit weight-only linear layer
 * y = x . dequant(W)^T for AMD Instinct MI355X (gfx950).
 *
 * The method (vibevoice.c README, section "Quantization" > "Weights"): each
 * projection weight W[N][K] (PyTorch Linear orientation, out x in) is cut
 * into blocks of 64 consecutive weights along K; every block keeps one
 * absmax scale s and every weight a 4-bit code into a 16-entry non-uniform
 * table c[] ("Int8 activations" section).  A weight reads back as c[idx]*s.
 * The decode GEMV and the prefill GEMM ("The kernels that matter": the
 * dequantization is fused into the multiply so the weights stay 4-bit into
 * the product) both read one shared repacked weight layout (same README,
 * "Quantization" > "Weights": one row-major layout permuted inside each
 * 16-byte run so one load feeds both the GEMV and the matrix-core operand).
 * A second 4-bit format, asymmetric int4 in groups of 128 with an integer
 * zero point (the nf4_awq_* entry points at the end), shares the layout and
 * the kernels.
 *
 * Conventions shared by every entry point
 *  - Every pointer except `codebook` is DEVICE memory owned by the caller.
 *    `codebook` is a HOST array of 16 floats, read during the call and baked
 *    into the kernel arguments (so a captured graph keeps its values).
 *  - Work is enqueued on `stream` only; nothing is allocated, freed or
 *    synchronised.  Passing 0 selects the null stream, which the library
 *    never picks by itself.
 *  - Arguments are validated on the host before any HIP call; a rejected call
 *    enqueues nothing.  A launch failure reported by hipGetLastError maps to
 *    NF4_ERR_HIP.  Device faults surface at the caller's next synchronisation.
 *  - The library holds no state: calls are reentrant and thread safe.
 *  - Shapes: N % 16 == 0, N >= 16; K % 64 == 0, K >= 64; 1 <= M <= 2^23.
 *    N, K <= 2^30 and N*K <= 2^40.
 *  - Device pointers must be 16-byte aligned (else NF4_ERR_ALIGN).
 *  - x is bfloat16 (hip_bfloat16: the 2-byte bit pattern), [M][K] row-major.  y is fp32 [M][N]
 *    row-major, overwritten (never accumulated), no bias.
 *
 * Device weight layout (what nf4_pack writes and the GEMV/GEMM read)
 *  - Rows are taken 16 at a time (row group g = n / 16) and K 128 at a time
 *    (tile t = k / 128; the last tile is zero-padded when K % 128 == 64).
 *    Tile (g, t) is 1024 bytes at byte offset (g * KT + t) * 1024 with
 *    KT = ceil(K / 128).
 *  - Inside a tile, 64 lanes own 16 bytes each at lane * 16.  Lane l holds
 *    row 16g + (l % 16); its dword j (0..3) holds the codes of
 *    k = 128t + 32j + 8(l / 16) + i, i = 0..7, code i in bits 4i..4i+3.
 *    Each dword is therefore four canonical bytes (low nibble = even k).
 *  - absmax: for tile (g, t), 32 floats at float offset (g * KT + t) * 32;
 *    entry 2r + h is the scale of row 16g + r, block 2t + h.
 *  - Padding codes are 0 and padding scales are +0.0.
 */
#ifndef NF4_H
#define NF4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_bfloat16.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nf4_status {
  NF4_OK = 0,
  NF4_ERR_NULL = 1,      /* a required pointer is NULL */
  NF4_ERR_SHAPE = 2,     /* M, N or K outside the limits above */
  NF4_ERR_ALIGN = 3,     /* a device pointer is not 16-byte aligned */
  NF4_ERR_CODEBOOK = 4,  /* codebook not usable by this entry point */
  NF4_ERR_WORKSPACE = 5, /* workspace smaller than nf4_workspace_bytes() */
  NF4_ERR_HIP = 6,       /* the HIP runtime rejected a launch */
  NF4_ERR_SCRATCH = 7    /* more scratch than nf4_gemv_argmax_noalloc holds */
} nf4_status;

/* Static string naming a status; never NULL. */
const char *nf4_status_string(nf4_status status);

/* Bytes of the device-layout code buffer: ceil(K/128) * (N/16) * 1024.
 * Returns 0 for shapes the library rejects. */
size_t nf4_qweight_bytes(int64_t N, int64_t K);

/* Bytes of the device-layout scale buffer: ceil(K/128) * (N/16) * 128.
 * Returns 0 for shapes the library rejects. */
size_t nf4_absmax_bytes(int64_t N, int64_t K);

/* Bytes of scratch that nf4_gemv / nf4_gemm need for an M x N x K call; the
 * larger of the two needs.  The GEMV sums its partials in LDS and needs
 * none.  The GEMM needs some only past 64 rows when it sums K in P > 1
 * parts (see nf4_gemm), which it runs on separate workgroups that meet
 * through the workspace: one 4-byte arrival counter per output tile of
 * 128 x 128, 128 x 224 or 128 x 256 (the largest need of the three tile
 * widths), then every part's sums of every tile (about 4 P M N bytes in
 * all).  0 otherwise, and the workspace arguments may then
 * be NULL with 0 bytes.  The workspace needs no initial contents: each call
 * that uses it first clears its counters with a small kernel on its stream.
 * Calls sharing one workspace must be ordered (one stream). */
size_t nf4_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* The default 16-entry codebook, computed on the host (no device work):
 * normal quantiles normalised to [-1, 1] with an exact zero (vibevoice.c
 * README, "Int8 activations: W8A8 and W4A8": NF4's codes index a
 * non-uniform table; "Quantization" > "Weights": NF4 blocks of 64 with
 * absmax scales).  With Phi the standard normal CDF and d = Phi^-1(delta):
 * 8 positive levels Phi^-1(1/2 + (delta - 1/2) j / 8) / d, j = 1..8, 7
 * negative levels -Phi^-1(1/2 + (delta - 1/2) j / 7) / d, j = 1..7, and +0.0,
 * sorted; each value rounded to the nearest bfloat16 (ties to even) and
 * stored as fp32, so c[0] = -1, c[7] = +0.0, c[15] = +1 and every product of
 * a bf16 activation with a code is exact in fp32.  delta = 0.9677083 gives
 * the table the rest of the library is measured with; any delta in
 * (0.75, 0.9999] is accepted (else NF4_ERR_CODEBOOK, nothing written).
 * codebook: host array of 16 floats, written. */
nf4_status nf4_codebook(double delta, float codebook[16]);

/* Quantize fp32 W[N][K] (row-major) into the device layout (vibevoice.c
 * README, "Quantization" > "Weights": blocks of 64 with an absmax scale
 * each, quantized deterministically once per projection at load, before
 * placement; the nearest-code rule and its tie-break are this library's
 * reading, which the page leaves open).  Per block of
 * 64: s = max |w| (exact); s == 0 gives every weight the index of the +0.0
 * code; otherwise idx = #{ i < 15 : (double)w > m_i * (double)s } with
 * m_i = ((double)c_i + (double)c_{i+1}) / 2, i.e. the nearest code with an
 * exact midpoint going to the lower index.  The codebook must be finite,
 * strictly increasing and contain +0.0 (else NF4_ERR_CODEBOOK).  W must be
 * finite (not checked).  qweight: nf4_qweight_bytes(N, K) bytes; absmax:
 * nf4_absmax_bytes(N, K) bytes. */
nf4_status nf4_pack(const float *W, int64_t N, int64_t K, const float codebook[16],
                    uint8_t *qweight, float *absmax, hipStream_t stream);

/* Debug path (vibevoice.c README, "Quantization" > "Weights": a weight reads
 * back as its code's table value times its block's absmax):
 * W_out[n][k] = fl32(c[idx] * s), one binary32 multiply per weight, fp32
 * [N][K] row-major.  Any finite codebook. */
nf4_status nf4_dequant(const uint8_t *qweight, const float *absmax, const float codebook[16],
                       int64_t N, int64_t K, float *W_out, hipStream_t stream);

/* Layout conversion from the canonical format (codes[N][K/2] bytes, byte j
 * = idx[2j] | idx[2j+1] << 4; scales[N][K/64] fp32 row-major) into the
 * device layout; for weights quantized elsewhere (vibevoice.c README,
 * "Quantization" > "Weights": checkpoints are repacked once at load into
 * one row-major layout whose 16-byte runs are permuted for the kernels). */
nf4_status nf4_repack(const uint8_t *codes, const float *scales, int64_t N, int64_t K,
                      uint8_t *qweight, float *absmax, hipStream_t stream);

/* Inverse of nf4_repack (same passage): device layout back to the
 * canonical format. */
nf4_status nf4_unpack(const uint8_t *qweight, const float *absmax, int64_t N, int64_t K,
                      uint8_t *codes, float *scales, hipStream_t stream);

/* Decode GEMV, 1 <= M <= 8 (vibevoice.c README, "The kernels that matter":
 * single-token decode reads every weight once and is bound by memory
 * bandwidth, with the dequantization fused into the multiply;
 * "Quantization" > "Weights", decode-GEMV bullet: 128-bit loads, same-input
 * projections in one launch):
 * y[m][n] = sum_b s[n][b] * sum_{k in b} x[m][k] * c[idx[n][k]], fp32
 * accumulation.  x: bfloat16 [M][K] row-major (hip_bfloat16 is the 2-byte
 * bit pattern).  y: fp32 [M][N] row-major, overwritten.  Codebook: any finite values whose fp32
 * entries are sums of at most three bfloat16 values (every normal fp32 is);
 * else NF4_ERR_CODEBOOK.  workspace: at least nf4_workspace_bytes(M, N, K)
 * bytes (any contents).  Results are bitwise reproducible run to run for a
 * given shape and device. */
nf4_status nf4_gemv(const hip_bfloat16 *x, int64_t M, const uint8_t *qweight, const float *absmax,
                    const float codebook[16], int64_t N, int64_t K, float *y, void *workspace,
                    size_t ws_bytes, hipStream_t stream);

/* nf4_gemv, plus a read-ahead hint naming the packed matrix of the next GEMV
 * launch on the stream (next_qweight, next_absmax, next_N x next_K, in the
 * device layout).  The pages put the shortfall of the small projections on
 * a fixed cost per kernel (vibevoice.c README, "Quantization" > "Weights",
 * the decode-GEMV bullet of the int4 GPU path: launch, ramp-up and tail); a
 * decode step knows its linears in advance, and a matrix does not depend on
 * activations, so this launch spends the loads it issues after its own
 * weights are in flight on the first tiles the next launch will read (as
 * planned for the same M), which then start from the caches.  y is computed
 * exactly as by nf4_gemv: bit for bit the same, with or without the hint.
 * next_qweight == NULL means no hint (next_absmax and the next shape are
 * then ignored).  Otherwise next_absmax must not be NULL, both must be
 * 16-byte aligned device buffers of an existing packed matrix whose shape
 * nf4_gemv accepts (else NF4_ERR_NULL, NF4_ERR_ALIGN, NF4_ERR_SHAPE); the
 * next matrix is only read.  Other arguments and errors as nf4_gemv. */
nf4_status nf4_gemv_prefetch(const hip_bfloat16 *x, int64_t M, const uint8_t *qweight,
                             const float *absmax, const float codebook[16], int64_t N, int64_t K,
                             float *y, void *workspace, size_t ws_bytes,
                             const uint8_t *next_qweight, const float *next_absmax,
                             int64_t next_N, int64_t next_K, hipStream_t stream);

/* Bytes of workspace nf4_gemv_argmax needs for an M x N x K call on the
 * current device: an arrival counter and one 8-byte candidate per workgroup
 * and row.  0 for shapes nf4_gemv rejects. */
size_t nf4_gemv_argmax_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Decode GEMV followed by the argmax of each output row: the step that turns
 * lm_head logits into the next token on the device (vibevoice.c README, "The
 * kernels that matter": the host then copies M indices instead of M x N
 * logits).  y is computed and written exactly as by nf4_gemv with the same
 * arguments; then index[m] = the smallest n with y[m][n] == max_n y[m][n],
 * compared as fp32 (NaN never wins; a row of NaN gives -1).  index: device
 * int32[M], 16-byte aligned.  workspace: at least
 * nf4_gemv_argmax_workspace_bytes(M, N, K) bytes, zero-filled once at
 * allocation; every call leaves its counter at zero, and calls sharing one
 * workspace must be ordered.  Errors as nf4_gemv, plus NF4_ERR_NULL for a
 * NULL index or workspace. */
nf4_status nf4_gemv_argmax(const hip_bfloat16 *x, int64_t M, const uint8_t *qweight,
                           const float *absmax, const float codebook[16], int64_t N, int64_t K,
                           float *y, int32_t *index, void *workspace, size_t ws_bytes,
                           hipStream_t stream);

/* nf4_gemv_argmax for callers that cannot allocate or pass a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels and results (y and index bit for bit those
 * of nf4_gemv_argmax with the same arguments), with the arrival counter and
 * candidates in a static device array of the library, 64 KiB per device,
 * held from the first call on a device until the process ends.  Each call
 * first clears the counter with a small kernel on `stream`, then runs the
 * GEMV + argmax; it calls no allocation routine.  Calls needing more than
 * 64 KiB (nf4_gemv_argmax_workspace_bytes(M, N, K) > 65536, i.e. more than
 * about 1000 workgroups' candidates; a 152064-row head at M = 8 on 256 CUs
 * needs 16.6 KB) return NF4_ERR_SCRATCH and enqueue nothing.  All calls of
 * a process on one device share the array: calls that overlap in time on
 * one device (two streams or two threads) race and must be ordered by the
 * caller.  The first call on a device looks up the array's
 * device address (NF4_ERR_HIP if that fails).  Other arguments and errors
 * as nf4_gemv_argmax. */
nf4_status nf4_gemv_argmax_noalloc(const hip_bfloat16 *x, int64_t M, const uint8_t *qweight,
                                   const float *absmax, const float codebook[16], int64_t N,
                                   int64_t K, float *y, int32_t *index, hipStream_t stream);

/* Prefill GEMM, any M >= 1 (vibevoice.c README, "Quantization" > "Weights",
 * M > 1 bullet: a matrix-core GEMM that keeps the weights 4-bit into on-chip
 * memory, expands them next to the matrix instruction, and splits K when the
 * grid would not cover the device, its partials in the caller's scratch):
 * same result definition as nf4_gemv, computed on
 * bf16 matrix cores with the codes as exact bf16 operands and the fp32
 * scales applied outside the matrix product once per 64-block.  The sum
 * over K runs in P parts, device tiles [b_j, b_j+1) with
 * b_j = ceil(j KT / P), KT = ceil(K/128): each part from zero in K order,
 * then the parts' sums added in part order.  P depends on N and K only:
 * P = 2 from K = 8192 on, else 1; then, when T P < 128 for
 * T = 8 ceil(N/128) (the 128 x 128 output tiles of a 1024-row batch),
 * P = max(P, min(256 / T, KT / 4)) (integer divisions).  workspace: at
 * least nf4_workspace_bytes(M, N, K) bytes, any contents (may be NULL when
 * that is 0), else NF4_ERR_NULL or NF4_ERR_WORKSPACE.  Results are
 * bitwise reproducible run to run, and a row of y does not depend on the
 * other rows of x; column slices of a matrix fused along N equal the
 * separate matrices' outputs bit for bit when both have the same P. */
nf4_status nf4_gemm(const hip_bfloat16 *x, int64_t M, const uint8_t *qweight, const float *absmax,
                    const float codebook[16], int64_t N, int64_t K, float *y, void *workspace,
                    size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Second weight format: asymmetric int4 in groups of 128 along K, with an
 * exact integer zero point per group (vibevoice.c README, "Quantization" >
 * "Weights": the INT4 option of the load-time quantizer, AWQ's own form, and
 * the AWQ/GPTQ repack paragraph, which reads a weight back as (q - z) * s
 * and keeps scale and zero point together, 4 bytes per group).  A weight
 * reads back as w = (q - z) * s with code q in 0..15, zero point z in 0..15
 * and a scale s that is a binary16 value, one (s, z) per row and group.
 * Here the product is exact (it always fits binary32); the pages' GPU
 * kernels round it to FP16.
 *
 * Shapes: as above, and K % 128 == 0 (one group per device tile row).
 * Device layout: the codes as in the NF4 layout above (dword j of lane l:
 * codes q of k = 128t + 32j + 8(l / 16) + i); params: for tile (g, t), 16
 * dwords at dword offset (g * KT + t) * 16, dword r = (binary16 bits of s)
 * | z << 16 for row 16g + r, group t.
 * ------------------------------------------------------------------------ */

/* Bytes of the params buffer: (N/16) * (K/128) * 64, or 0 when K % 128 != 0
 * or the shape is rejected.  The code buffer is nf4_qweight_bytes(N, K). */
size_t nf4_awq_params_bytes(int64_t N, int64_t K);

/* Bytes of workspace nf4_awq_gemm (and nf4_awq_gemv when x does not fit its
 * on-chip path) needs: K/128 x (M rounded up to 128) floats, the sums of x
 * over every 128-k group; past 64 rows with K in P > 1 parts (nf4_gemm's
 * rule) also the arrival counters and part sums (nf4_workspace_bytes'
 * layout).  0 for shapes these calls reject.  Every call sets what it reads (the
 * counters included) itself, so the workspace needs no initial contents;
 * calls sharing one must be ordered. */
size_t nf4_awq_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Quantize fp32 W[N][K] (row-major, finite) into the device layout.  Per row
 * and group of 128 (lo = min w, hi = max w, computed in double):
 * s = fp16(max(hi - lo, 1e-5) / 15) (nearest binary16, ties to even;
 * +inf past the binary16 range), z = clamp(rint(-lo / s), 0, 15),
 * q = clamp(rint(w / s) + z, 0, 15), with rint rounding ties to even and
 * every division in double.  qweight: nf4_qweight_bytes(N, K) bytes; params:
 * nf4_awq_params_bytes(N, K) bytes. */
nf4_status nf4_awq_pack(const float *W, int64_t N, int64_t K, uint8_t *qweight,
                        uint32_t *params, hipStream_t stream);

/* Layout conversion for weights quantized elsewhere: codes[N][K/2] (byte j =
 * q[2j] | q[2j+1] << 4), scales[N][K/128] binary16 bit patterns, zeros
 * [N][K/128] bytes (the low 4 bits are used), all row-major device arrays
 * (16-byte aligned), into the device layout.  Values are taken as given. */
nf4_status nf4_awq_repack(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                          int64_t N, int64_t K, uint8_t *qweight, uint32_t *params,
                          hipStream_t stream);

/* Inverse of nf4_awq_repack: device layout back to codes, scales (binary16
 * bits) and zero points, same arrays and alignment. */
nf4_status nf4_awq_unpack(const uint8_t *qweight, const uint32_t *params, int64_t N, int64_t K,
                          uint8_t *codes, uint16_t *scales, uint8_t *zeros, hipStream_t stream);

/* Debug path: W_out[n][k] = fl32((q - z) * s) (exact), fp32 [N][K]
 * row-major. */
nf4_status nf4_awq_dequant(const uint8_t *qweight, const uint32_t *params, int64_t N, int64_t K,
                           float *W_out, hipStream_t stream);

/* Activation gather for act-order checkpoints (vibevoice.c README,
 * "Quantization" > "Weights", the GPTQ act-order bullet): such checkpoints
 * quantized the input channels in order of importance, so a group's channels
 * are scattered over K.  Sorting the channels by group at load (a stable sort
 * of the per-channel group index; perm[j] = the j-th channel) makes every
 * group a contiguous run that nf4_awq_pack / nf4_awq_repack and the linears
 * take as is, and the decoder then gathers x through the same order before
 * the product: x_out[m][j] = x[m][perm[j]] (bf16 bit patterns, [M][K]
 * row-major).  perm: device int32[K]; values outside [0, K) are clamped into
 * it.  1 <= M <= 2^23, K % 8 == 0 (else NF4_ERR_SHAPE); x, perm and x_out
 * 16-byte aligned device buffers; x_out must not overlap x. */
nf4_status nf4_gather_columns(const hip_bfloat16 *x, int64_t M, int64_t K, const int32_t *perm,
                              hip_bfloat16 *x_out, hipStream_t stream);

/* Decode GEMV of the int4 format, 1 <= M <= 8:
 * y[m][n] = sum_t s[n][t] * sum_{k in group t} x[m][k] * (q[n][k] - z[n][t]),
 * fp32 accumulation: per group the matrix cores add the exact products
 * x * q to -z * X (X = the group's sum of x, fp32), and the scale multiplies
 * that once.  workspace: may be NULL with 0 bytes when x fits the on-chip
 * path (M * K * 2 bytes of x plus K/4 bytes of sums within a workgroup's
 * 160 KB of LDS, about M * K <= 78000); otherwise the call runs the GEMM of
 * nf4_awq_gemm and needs nf4_awq_workspace_bytes(M, N, K) bytes (else
 * NF4_ERR_NULL or NF4_ERR_WORKSPACE).  Bitwise reproducible run to run. */
nf4_status nf4_awq_gemv(const hip_bfloat16 *x, int64_t M, const uint8_t *qweight,
                        const uint32_t *params, int64_t N, int64_t K, float *y, void *workspace,
                        size_t ws_bytes, hipStream_t stream);

/* nf4_awq_gemv plus the read-ahead hint of nf4_gemv_prefetch: the packed
 * int4 matrix of the next GEMV launch on the stream (next_qweight,
 * next_params, next_N x next_K), whose first tiles this launch loads after
 * its own weights are in flight.  y is bit for bit that of nf4_awq_gemv.
 * next_qweight == NULL means no hint; otherwise next_params must not be NULL,
 * both 16-byte aligned, and the next shape one that nf4_awq_gemv accepts
 * (else NF4_ERR_NULL, NF4_ERR_ALIGN, NF4_ERR_SHAPE).  The hint is ignored
 * when this call runs the GEMM path. */
nf4_status nf4_awq_gemv_prefetch(const hip_bfloat16 *x, int64_t M, const uint8_t *qweight,
                                 const uint32_t *params, int64_t N, int64_t K, float *y,
                                 void *workspace, size_t ws_bytes, const uint8_t *next_qweight,
                                 const uint32_t *next_params, int64_t next_N, int64_t next_K,
                                 hipStream_t stream);

/* Prefill GEMM of the int4 format, any M >= 1: the result definition of
 * nf4_awq_gemv on the tiled matrix-core kernel, after a pre-pass that writes
 * the group sums of x into the workspace (nf4_awq_workspace_bytes(M, N, K)
 * bytes, required).  K is summed in the parts nf4_gemm uses.  Rows of y do not depend on the other rows of x.  Shapes
 * whose byte offsets into x, qweight or the workspace reach 2^32 give
 * NF4_ERR_SHAPE.  Bitwise reproducible run to run. */
nf4_status nf4_awq_gemm(const hip_bfloat16 *x, int64_t M, const uint8_t *qweight,
                        const uint32_t *params, int64_t N, int64_t K, float *y, void *workspace,
                        size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NF4_H */
