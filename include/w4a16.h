/*
 * w4a16.h -- C ABI of libw4a16.so: batch-1 (M <= 8) matrix-vector product
 * y = W x with 4-bit weights, dequantized inside the kernel (W4A16 GEMV),
 * for AMD Instinct MI355X (gfx950); with it the host packer and quantizer,
 * a split-K GEMV, the fused gate/up + SwiGLU GEMV, an INT8-activation
 * variant, a matrix-core GEMM for many activation rows (prefill) and
 * standalone dequantization.
 *
 * The operation. W is N x K (N output features, K input features, row-major
 * like the matrix of the row-per-output GEMV of "CodeAlign-Runtime", Level 1).
 * Every run of 128 consecutive weights along K in one row is a group g with
 * one fp16 scale s[n][g] and one 4-bit zero point z[n][g]; weight values q are
 * unsigned 4-bit integers and
 *     w[n][k] = (q[n][k] - z[n][g]) * s[n][g],   g = k / 128
 * ("Building an LLM Inference Runtime ... Qwen2.5-Coder-7B on NVIDIA H100",
 * section "The Stack Architecture": one fp16 scale per group of 128 per
 * output row; "CodeAlign-Runtime", Level 3, "Quantization Scheme"). The
 * pages' signed symmetric format (two's-complement nibble t, zero point 0)
 * is the special case q = t xor 8, z = 8. Activations x are fp16 [M][K]
 * row-major, products accumulate in fp32, and y is fp16 [M][N] row-major,
 * rounded to nearest even:
 *     y[m][n] = sum_k w[n][k] * x[m][k].
 * The weights are never materialised: dequantization happens in registers
 * ("CodeAlign-Runtime", Level 3).
 *
 * Conventions for every entry point:
 *  - Return 0 (W4A16_OK) or a negative W4A16_E* code; nothing throws.
 *  - The caller owns every buffer: host memory for pack/unpack, device memory
 *    for the rest. The library never allocates, frees or synchronizes.
 *  - Device entry points are asynchronous on `stream` (a hipStream_t; NULL is
 *    the null stream). Faults during execution surface at the caller's next
 *    synchronization. They do no host synchronization, allocation or
 *    host read of device memory, so they can be captured into a hipGraph.
 *  - Shapes: K must be a multiple of 128 and >= 128; 1 <= M <= 8 for the
 *    GEMV entry points. M == 0 or N == 0 is a valid empty call: it returns
 *    W4A16_OK without touching any pointer and without launching.
 *  - Device pointers must be 16-byte aligned. Outputs of a call that
 *    returns an error are unspecified.
 *  - No global state but the per-GPU accumulation array of
 *    w4a16_gemv_splitk_noalloc (calls to that entry point on one GPU must be
 *    ordered); every other entry point is reentrant.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_OK 0
#define W4A16_EINVAL (-1)      /* bad shape, null or misaligned pointer, bad value */
#define W4A16_EUNSUPPORTED (-2) /* M > 8 for a GEMV (w4a16_gemm serves more rows), or a shape
                                   outside what an entry point documents it supports */
#define W4A16_ELAYOUT (-3)     /* layout ID mismatch (see w4a16_layout_id) */
#define W4A16_EHIP (-4)        /* the HIP runtime refused a launch */

#define W4A16_GROUP 128
#define W4A16_MAX_M 8

/*
 * Layout identifier of the packed buffers this library reads and writes: 2.
 * The runtime only ever understands this one layout, fixed with the packer
 * (the practice of "Building an LLM Inference Runtime", Bug #3, where the
 * runtime refuses weights of any other layout ID). Layout ID 2, for N x K:
 *   NP = N rounded up to 16, G = K/128. Tile (t, g) is rows 16t .. 16t+15
 *   of group g; all three buffers list tiles in the order t*G + g.
 *   Wq: NP/16 * G tiles of 1024 bytes, tile (t, g) at byte (t*G + g)*1024.
 *     The little-endian 32-bit word at byte lane*16 + kb*4 of a tile
 *     (lane in [0,64), kb in [0,4)) holds row 16t + lane%16, columns
 *     k = 128g + 32kb + 8*(lane/16) + j (j in [0,8)), weight j in bits
 *     4*SLOT[j] .. 4*SLOT[j]+3 with SLOT = {0,4,1,5,2,6,3,7} -- the
 *     ValueShuffle interleave of that page, which is also AWQ's
 *     interleaved order ("Custom AWQ Dequantization Kernel", Part 2).
 *   scales: 16 fp16 per tile, row n group g at element (t*G + g)*16 + n%16
 *     (t = n/16): NP*G*2 bytes.
 *   zeros: 16 nibbles per tile, row n group g in byte (t*G + g)*8 + (n%16)/2,
 *     low nibble for even n, high nibble for odd n: NP*G/2 bytes.
 *   Padding rows (n >= N) are zero in all three buffers.
 */
int w4a16_layout_id(void);

/*
 * Host: the loader's check of the layout ID stored with a set of packed
 * weights (for example in its weight file's header), refusing any layout
 * but this library's as the runtime of "Building an LLM Inference Runtime"
 * does (Bug #3). Returns W4A16_OK for layout_id == w4a16_layout_id(), else
 * W4A16_ELAYOUT. Packed buffers themselves carry no tag: their sizes are
 * exactly those of w4a16_packed_sizes.
 */
int w4a16_check_layout(int layout_id);

/*
 * Sizes in bytes of the three packed buffers for an N x K matrix.
 * N >= 0; K a multiple of 128 and >= 128. Any of the size pointers may be
 * NULL. Errors: W4A16_EINVAL for a bad shape.
 */
int w4a16_packed_sizes(int N, int K, size_t* wq_bytes, size_t* s_bytes, size_t* z_bytes);

/*
 * Host packer: logical tensors -> layout ID 2 (host memory to host memory).
 *   q  [N][K]    uint8, each 0..15 (the 4-bit weights)
 *   s  [N][K/128] uint16, fp16 bit patterns (any pattern is accepted)
 *   z  [N][K/128] uint8, each 0..15 (the zero points)
 *   wq_out, s_out, z_out: caller buffers of w4a16_packed_sizes() bytes;
 *   they are overwritten entirely, padding included.
 * Errors: W4A16_EINVAL for a bad shape, a NULL pointer (when N > 0), or a
 * q or z value above 15. Runs on the calling thread (no GPU needed).
 */
int w4a16_pack(int N, int K, const uint8_t* q, const uint16_t* s, const uint8_t* z,
               void* wq_out, void* s_out, void* z_out);

/*
 * Host packer for the fused gate/up + SwiGLU GEMV (w4a16_gemv_swiglu).
 * Gate and up are two F x K matrices in the logical form of w4a16_pack
 * (qg, sg, zg and qu, su, zu). They are interleaved in blocks of 8 rows --
 * gate rows 8j .. 8j+7, then the up rows 8j .. 8j+7, so that each 16-row
 * tile of the layout holds both projections of 8 outputs -- into one
 * matrix of 16 * ceil(F/8) rows (rows past F within a tile are zero),
 * which is packed as by w4a16_pack. That interleave is what lets SwiGLU run
 * in registers (the 4-bit matrix-vector kernel of the qengine page, "How it
 * works"). Output buffers: w4a16_packed_sizes(16 * ceil(F/8), K) bytes.
 * Errors: as w4a16_pack, and W4A16_EINVAL when 16 * ceil(F/8) exceeds
 * INT32_MAX. Host only; allocates nothing.
 */
int w4a16_pack_gate_up(int F, int K, const uint8_t* qg, const uint16_t* sg, const uint8_t* zg,
                       const uint8_t* qu, const uint16_t* su, const uint8_t* zu, void* wq_out, void* s_out,
                       void* z_out);

/*
 * Host round-to-nearest quantizer: fp16 weights w [N][K] (bit patterns,
 * row-major, all finite) -> the logical q [N][K], s [N][K/128] (fp16 bits)
 * and z [N][K/128] that w4a16_pack takes. Each group of 128 consecutive
 * weights of a row gets its own scale; values are computed in double
 * precision, codes divide by the stored fp16 scale and round half to even.
 *   mode 0, symmetric, the scheme of "Building an LLM Inference Runtime",
 *     "The Stack Architecture" and "CodeAlign-Runtime", Level 3:
 *     s = fp16(absmax / 7), t = clamp(round(w / s), -8, 7), stored as
 *     q = t + 8 with z = 8, so (q - z) * s = t * s.
 *   mode 1, asymmetric, for uint4 zero points: with lo = min(w, 0) and
 *     hi = max(w, 0) over the group, s = fp16((hi - lo) / 15),
 *     z = clamp(round(-lo / s), 0, 15), q = clamp(round(w / s) + z, 0, 15).
 *   A group whose scale rounds to 0 gets q = z (it dequantizes to 0).
 * Errors: W4A16_EINVAL for a bad shape or mode, a NULL pointer (when N > 0)
 * or a non-finite weight. Runs on host threads (no GPU needed); where a
 * thread cannot be started, its rows run on the calling thread.
 */
int w4a16_quantize(int N, int K, const uint16_t* w, int mode, uint8_t* q, uint16_t* s, uint8_t* z);

/*
 * Inverse of w4a16_pack (host to host): recovers q [N][K], s [N][K/128] and
 * z [N][K/128] exactly. Errors: W4A16_EINVAL for a bad shape or NULL pointer.
 */
int w4a16_unpack(int N, int K, const void* wq, const void* s_packed, const void* z_packed,
                 uint8_t* q, uint16_t* s, uint8_t* z);

/*
 * y = W x on the GPU (the hot path).
 *   M: activation rows, 1..8 (a decode token plus speculative drafts);
 *   N, K: weight shape (K multiple of 128); Wq, scales, zeros: device
 *   buffers in layout ID 2; x: device fp16 [M][K]; y: device fp16 [M][N].
 * Each output is a fixed-order fp32 sum (no atomics): repeated calls give
 * bit-identical results. Errors: W4A16_EINVAL (shape, NULL, alignment),
 * W4A16_EUNSUPPORTED (M > 8), W4A16_EHIP (launch refused).
 */
int w4a16_gemv(int M, int N, int K, const void* Wq, const void* scales, const void* zeros,
               const void* x, void* y, void* stream);

/*
 * Fused gate/up GEMV with a SwiGLU epilogue:
 *   y[m][f] = fp16( silu(g) * u ),  g = sum_k Wgate[f][k] x[m][k],
 *   u = sum_k Wup[f][k] x[m][k],  silu(g) = g / (1 + exp(-g)),
 * with g and u the fp32 sums of the GEMV (never rounded to fp16) and the
 * epilogue evaluated in fp32. Wq, scales, zeros: the interleaved matrix
 * written by w4a16_pack_gate_up, on the device. x: fp16 [M][K];
 * y: fp16 [M][F]. M: 1..8. The SwiGLU activation is the one of the Qwen2.5
 * MLP the pages' 7B shapes come from; its placement in registers, right
 * after the gate and up sums, follows the qengine page ("How it works").
 * Saves the separate activation launch and the 2 * M * 2F bytes of the
 * intermediate gate/up output. Each tile's gate and up sums are the
 * plain GEMV's sums of its rows (the same waves and shares as w4a16_gemv
 * on the packed matrix), so the call is deterministic and batch invariant
 * like w4a16_gemv and takes any K it takes. Errors: as w4a16_gemv, and
 * W4A16_EUNSUPPORTED when 16 * ceil(F/8) exceeds INT32_MAX.
 */
int w4a16_gemv_swiglu(int M, int F, int K, const void* Wq, const void* scales, const void* zeros,
                      const void* x, void* y, void* stream);

/*
 * Workspace bytes w4a16_gemv_splitk needs for an M x N output: one uint64
 * accumulation word per output, 8 * M * N rounded up to a multiple of 16
 * (the same for every split count). Returns 0 for a negative argument.
 */
size_t w4a16_splitk_workspace_bytes(int M, int N, int splits);

/*
 * Split count this library recommends for an M x N x K split-K call,
 * measured on MI355X: about one split per 16 groups of 128 when K has at
 * least 96 groups and the matrix 257 to 1023 tiles of 16 rows; about one
 * per 12 groups when it has fewer than 128 tiles and K at least 24 groups;
 * 2 when it has 1024 to 2047 tiles and K at least 40 groups; otherwise 1
 * (do not split). At most 16. It does not depend on M, so rows stay batch
 * invariant for a caller who follows it. Returns 0 for an invalid shape.
 */
int w4a16_splitk_choose(int M, int N, int K);

/*
 * Split-K variant of w4a16_gemv for long K. The K groups are divided into
 * `splits` contiguous ranges, so a matrix with few rows still gets a grid
 * large enough to fill the GPU. This is the two-stage partial/final shape of
 * "CodeAlign-Runtime", Level 4, applied to K, done in one launch:
 *   - each (16-row tile, range) workgroup turns its fp32 partial sums into
 *     fixed point, round(p * 2^24), and adds them with a device-scope atomic
 *     to one 64-bit word per output in `workspace`;
 *   - the word also counts the arrivals, so the add that completes the count
 *     returns the whole sum; that workgroup writes y = fp16(sum * 2^-24) and
 *     sets the word back to zero.
 * Integer addition is exact and order-free, so results are bit-identical run
 * to run whatever the arrival order (the determinism rule of the qengine
 * page, "Learnings": float atomics made runs differ). Each fixed-point
 * partial is within 2^-25 of the fp32 one; a partial is clamped to
 * |p| < 2^29 (past that the workload's error bound already exceeds the whole
 * fp16 range, and a clamped sum still overflows to +-inf in fp16 as the
 * exact one would), and a NaN partial counts as 0. No workgroup ever waits
 * for another, and no fence is needed: each word is one atomic location.
 *   1 <= splits <= min(K/128, 31); splits == 1 is w4a16_gemv and does not
 *   touch the workspace.
 *   workspace: device memory, 16-byte aligned, at least
 *   w4a16_splitk_workspace_bytes(M, N, splits) bytes, zero-filled once
 *   before its first use. Every completed call leaves it all zero again, so
 *   one workspace serves any later call on the same stream, and graph
 *   replays too. Calls that may overlap in time (different streams) need
 *   different workspaces.
 * Results may differ in rounding from w4a16_gemv (another summation order)
 * but lie within the same accuracy bound. Errors are as w4a16_gemv, plus
 * W4A16_EINVAL for a bad split count or a short workspace.
 */
int w4a16_gemv_splitk(int M, int N, int K, int splits, const void* Wq, const void* scales,
                      const void* zeros, const void* x, void* y, void* workspace, size_t ws_bytes,
                      void* stream);

/*
 * Bytes of the device array behind w4a16_gemv_splitk_noalloc: 2 MiB per GPU,
 * one uint64 accumulation word per output, so M * N <= 262144.
 */
#define W4A16_NOALLOC_SCRATCH_BYTES (2u << 20)

/*
 * w4a16_gemv_splitk for callers that cannot allocate device memory (code
 * under graph capture, serving loops or harnesses that forbid hipMalloc):
 * the same split-K GEMV, with the same plan and kernel and so the same bits,
 * but its accumulation words live in a file-scope device array of the
 * library (W4A16_NOALLOC_SCRATCH_BYTES per GPU, held by each GPU the library
 * runs on until the process ends) instead of a caller workspace. The caller
 * still passes the inputs and the output. The call allocates nothing: no
 * hipMalloc, hipFree or allocating library routine. The first call on a
 * device looks the array up (hipGetSymbolAddress, with that device current)
 * and clears it with a fill kernel on `stream`; every completed call leaves
 * it zero again. Calls on one GPU share that GPU's array: calls that overlap
 * in time on one GPU (different streams, or different host threads without
 * ordering) race and give wrong results; order them on one stream.
 *   M, N, K, splits, Wq, scales, zeros, x, y: as w4a16_gemv_splitk;
 *   splits == 1 is w4a16_gemv and does not touch the array.
 * Errors: as w4a16_gemv_splitk; W4A16_EUNSUPPORTED when M * N exceeds
 * W4A16_NOALLOC_SCRATCH_BYTES / 8 (use w4a16_gemv_splitk with a workspace);
 * W4A16_EHIP when the array cannot be looked up or cleared.
 */
int w4a16_gemv_splitk_noalloc(int M, int N, int K, int splits, const void* Wq, const void* scales,
                              const void* zeros, const void* x, void* y, void* stream);

/*
 * W4A16 GEMM for many activation rows (prefill, M > 8), on the matrix cores:
 * y[M][N] = x[M][K] W^T. Wq, scales, zeros: device buffers in layout ID 2;
 * x: device fp16 [M][K]; y: device fp16 [M][N]; any M >= 1 (for M <= 8
 * w4a16_gemv is the faster path). The weights are dequantized in registers
 * to fp16 (q - z) * s, each rounded once to nearest even (the values
 * w4a16_dequant_f16 writes), and multiplied with fp32 accumulation; the
 * products are exact, so each output is within fp32 accumulation and fp16
 * output rounding of sum_k fp16w * x -- inside the workload's bound
 * 2e-3 * sum|w x| + 1e-5, the weight rounding taking at most 2^-11 of it.
 * A workgroup covers 16, 32, 64 or 128 rows of x (the fewest of these that
 * cover M; above 64 rows, 64 where the grid of 64-row tiles holds at most
 * 256 workgroups, or where M is 129 .. 192, and 128 otherwise)
 * and 128 of W. Each output's sum is the same sequence of products for
 * every tile height, so row m of the result does not depend on M.
 * Deterministic (fixed order), but not bit-equal to w4a16_gemv, whose
 * weights are exact (q - z) scaled per group. The standalone dequant + MFMA
 * GEMM variant the AWQ dequantization page builds in two steps, here in
 * one. Errors: W4A16_EINVAL (shape, NULL, alignment), W4A16_EUNSUPPORTED
 * (K >= 2^25), W4A16_EHIP.
 */
int w4a16_gemm(int M, int N, int K, const void* Wq, const void* scales, const void* zeros, const void* x,
               void* y, void* stream);

/*
 * INT8 activations, step 1 of 2: the activation quantizer of the alternative
 * path ("Path A") of "Building an LLM Inference Runtime", Bug #3, which turns
 * the fp16 activations into 8-bit integers with one scale per group in a
 * launch of its own before each GEMV. Per activation row m and group g of 128
 * consecutive columns (the weight groups' column ranges):
 *     sx[m][g]   = absmax_g / 127            (fp32, correctly rounded)
 *     xq[m][k]   = clamp(rne(x[m][k] / sx[m][g]), -127, 127)   (fp32 division)
 *     xsum[m][g] = sum of the group's codes
 * and a group of zeros gets sx = 0 and codes 0. x: device fp16 [M][K]
 * (finite values; codes for NaN or infinity are unspecified); xq: device
 * int8 [M][K]; sx: device fp32 [M][K/128]; xsum: device int32 [M][K/128],
 * all row-major and 16-byte aligned. Same M and K rules as w4a16_gemv.
 * Errors: W4A16_EINVAL (shape, NULL, alignment), W4A16_EUNSUPPORTED (M > 8),
 * W4A16_EHIP.
 */
int w4a16_act_quant_i8(int M, int K, const void* x, void* xq, void* sx, void* xsum, void* stream);

/*
 * INT8 activations, step 2 of 2: the GEMV over the codes of
 * w4a16_act_quant_i8, on the integer matrix cores (the counterpart of the
 * page's dp4a):
 *     y[m][n] = sum_g s[n][g] * sx[m][g] * sum_{k in g} (q[n][k] - z[n][g]) * xq[m][k]
 * Each group's integer sum is exact (computed as sum q xq - z * xsum); the
 * group terms are scaled and summed in fp32, in a fixed order, and y is
 * rounded to fp16 (nearest even): within 2e-3 * sum_g |term| + 1e-5 of the
 * exact value. This approximates w4a16_gemv's y by the activation rounding
 * (at most sum_g s * sx / 2 * sum_k |q - z| per output); it is provided for
 * comparison, as on that page. Wq, scales, zeros: layout ID 2; xq, sx, xsum:
 * the outputs of w4a16_act_quant_i8 for the same M and K; y: device fp16
 * [M][N]. Rows are bit-identical whatever M. Errors: as w4a16_gemv.
 */
int w4a16_gemv_a8(int M, int N, int K, const void* Wq, const void* scales, const void* zeros, const void* xq,
                  const void* sx, const void* xsum, void* y, void* stream);

/*
 * w4a16_act_quant_i8 and w4a16_gemv_a8 in one launch: x is fp16 [M][K] as
 * for w4a16_gemv, and each workgroup quantizes the activation groups it
 * multiplies (per group of 128: sx = absmax / 127, codes rne(x / sx)
 * clamped to +-127, their sum) with the same fp32 operations as
 * w4a16_act_quant_i8, so y equals that two-launch path bit for bit, with no
 * code buffers and one dependent launch fewer per GEMV. Same M limit, same
 * bound and batch invariance as w4a16_gemv_a8. Errors: W4A16_EINVAL (shape,
 * NULL, alignment), W4A16_EUNSUPPORTED (M > 8), W4A16_EHIP.
 */
int w4a16_gemv_a8_fused(int M, int N, int K, const void* Wq, const void* scales, const void* zeros, const void* x,
                        void* y, void* stream);

/*
 * Split count this library recommends for w4a16_gemm_splitk (1: do not
 * split), measured on MI355X over the 7B-shaped matrices at M = 1 .. 2048.
 * With B the workgroup's rows (16, 32, 64 or 128: the fewest of these that
 * cover M) and W the number of B x 128 output tiles: 1 from 256 tiles on;
 * where K holds >= 96 groups, min(8, 256 / W), or min(16, 512 / W) for
 * B = 16, and 3 where that gives 1 and 3 W <= 512; where it holds fewer, 4 if W <= 40 and M <= 96 (or W <= 32 and
 * M <= 128), else 1 (each split adds a pass of atomics over its tile, which
 * a short K does not pay for once the tile holds many rows); never above
 * K/512 or 31. It depends on M, and the GEMM makes no batch-invariance
 * promise. Returns 0 for an invalid shape or one w4a16_gemm does not
 * support.
 */
int w4a16_gemm_splitk_choose(int M, int N, int K);

/*
 * w4a16_gemm with the K groups divided into `splits` contiguous ranges, so
 * that a product with few output tiles (few rows, or a narrow matrix with a
 * long K) still fills the GPU. Each (tile, range) workgroup
 * adds its fp32 partial sums to one 64-bit fixed-point word per output, and
 * the add that completes an output's count writes y, exactly as in
 * w4a16_gemv_splitk (same format, same error: each partial within 2^-25 of
 * its fp32 value; results bit-identical run to run, whatever the arrival
 * order; within the workload's bound). The workspace rules are those of
 * w4a16_gemv_splitk: device memory, 16-byte aligned, at least
 * w4a16_splitk_workspace_bytes(M, N, splits) bytes, zero-filled once before
 * its first use and left zero by every completed call; calls that may
 * overlap in time need different workspaces. 1 <= splits <= min(K/128, 31);
 * splits == 1 is w4a16_gemm and does not touch the workspace. Errors: as
 * w4a16_gemm, plus W4A16_EINVAL for a bad split count or a short workspace.
 */
int w4a16_gemm_splitk(int M, int N, int K, int splits, const void* Wq, const void* scales, const void* zeros,
                      const void* x, void* y, void* workspace, size_t ws_bytes, void* stream);

/*
 * Bytes of the fp32 partials buffer w4a16_gemm_splitk_partials needs for an
 * M x N output in `splits` ranges: 4 * splits * M * N, rounded up to a
 * multiple of 16. Returns 0 for a negative size or splits < 1.
 */
size_t w4a16_gemm_partials_bytes(int M, int N, int splits);

/*
 * Split count this library recommends for w4a16_gemm_splitk_partials (1: do
 * not split). With W the output tiles of a split launch (128 columns by 16,
 * 32, 64 or 128 rows, the fewest that cover M): none from 256 tiles on; else
 * about 160 workgroups in all, more for a long K (toward 20 groups of K per
 * range while the grid stays within 256 workgroups); at least 4 groups of K
 * per range, at most 16 ranges. Returns 0 for an invalid shape or one
 * w4a16_gemm does not support.
 */
int w4a16_gemm_partials_choose(int M, int N, int K);

/*
 * w4a16_gemm with K divided into `splits` contiguous ranges, combined in two
 * stages ("CodeAlign-Runtime", Level 4: partial sums, then one final
 * reduction) instead of by atomics: each (tile, range) workgroup stores its
 * fp32 partial sums to partials[z][M][N] (z = the range), and a second
 * launch on the same stream writes y[m][n] = fp16(partials[0][m][n] + ... +
 * partials[splits-1][m][n]), added in range order in fp32. Deterministic
 * (bit-identical run to run) and within the workload's bound; not
 * bit-identical to w4a16_gemm_splitk, whose exact fixed-point combine
 * rounds differently. The atomics that combine costs grow with M * N *
 * splits; these plain stores and the final pass do not, so narrow matrices
 * at prefill sizes (M = 16 .. 384) split further for the same price.
 * partials: device memory, 16-byte aligned, at least
 * w4a16_gemm_partials_bytes(M, N, splits) bytes, needing no initial contents
 * (every element is written before it is read); calls that may overlap in
 * time need different buffers. 1 <= splits <= min(K/128, 31); splits == 1
 * is w4a16_gemm and does not touch the buffer. Errors: as w4a16_gemm, plus
 * W4A16_EINVAL for a bad split count, a NULL or misaligned buffer, or one
 * shorter than w4a16_gemm_partials_bytes.
 */
int w4a16_gemm_splitk_partials(int M, int N, int K, int splits, const void* Wq, const void* scales,
                               const void* zeros, const void* x, void* y, void* partials, size_t partials_bytes,
                               void* stream);

/*
 * Standalone dequantization, for paths that want the fp16 matrix itself
 * (a GEMM over many activation rows, for instance): W_out[n][k] =
 * fp16((q - z) * s), the exact product rounded once to nearest even, for
 * n < N, k < K. W_out: device fp16 [N][K] row-major, 16-byte aligned. This
 * is the dequantize entry point of "Custom AWQ Dequantization Kernel" for
 * layout 2. Errors: W4A16_EINVAL (shape, NULL, alignment), W4A16_EHIP.
 */
int w4a16_dequant_f16(int N, int K, const void* Wq, const void* scales, const void* zeros, void* W_out,
                      void* stream);

/*
 * Test hook: W_out[n][k] = float(q - z) * float(s) for n < N, k < K (device
 * fp32 [N][K] row-major), computed with the same in-register unpack as the
 * GEMV. The product is exact in fp32 (|q - z| <= 15 needs 4 bits, s has an
 * 11-bit significand), so the result is comparable bit for bit. This is the
 * dequantize entry point of "Custom AWQ Dequantization Kernel" for layout 2.
 * Errors: W4A16_EINVAL (shape, NULL, alignment), W4A16_EHIP.
 */
int w4a16_dequant_f32(int N, int K, const void* Wq, const void* scales, const void* zeros,
                      float* W_out, void* stream);

/*
 * Measurement hook: reads the `bytes` bytes at `buf` (device memory) once,
 * with the GEMV's non-temporal 16-byte loads, `grid` workgroups of 256
 * threads striding over them, and stores nothing but possibly one 32-bit
 * word of `sink` (device memory, 16 bytes). Its time gives the plain-read
 * ceiling of the device, the figure the GEMV's bandwidth is compared with
 * besides the specified peak. buf and sink 16-byte aligned, bytes a
 * multiple of 16, 1 <= grid <= 65535. Errors: W4A16_EINVAL, W4A16_EHIP.
 */
int w4a16_read_probe(const void* buf, size_t bytes, int grid, void* sink, void* stream);

/*
 * A chain of dependent GEMVs in one launch -- a whole decode step's linear
 * layers, each reading an earlier GEMV's output -- so that no launch
 * boundary stops the weight stream between them. The qengine page runs its
 * matrix kernels at 94.9% of bandwidth inside its decode loop by starting
 * each kernel's loads before the previous kernel finishes ("Why speed is a
 * byte count", "How it works"); here every workgroup requests the weights
 * of its next work items before it waits for their input.
 *
 * One GEMV of the chain:
 *   kind   W4A16_CHAIN_GEMV: y = W x as w4a16_gemv / w4a16_gemv_splitk;
 *          W4A16_CHAIN_SWIGLU: y = silu(gate x) * (up x) as
 *          w4a16_gemv_swiglu (W from w4a16_pack_gate_up, N = F, the output
 *          width; splits 1).
 *   N, K   output and input features (K a multiple of 128, at most 32768:
 *          each workgroup holds a GEMV's whole input in LDS).
 *   splits K ranges combined by the split-K fixed-point atomics (1..31).
 *          A wave takes its share of a range in rounds of at most 7 tiles
 *          (16 x 128 weights each).
 *   x_src  -1: the input is `x`, fp16 [M][K] on the device; otherwise the
 *          index of an earlier GEMV of the chain whose output has at least K
 *          columns: the input is its first K columns, times 2^-x_shift
 *          (0 <= x_shift <= 24; an exact power-of-two rescale, then fp16
 *          rounding to nearest even).
 *   wq, scales, zeros: layout ID 2 on the device; y: fp16 [M][N] on the
 *          device, written for every GEMV. 16-byte aligned.
 */
#define W4A16_CHAIN_GEMV 0
#define W4A16_CHAIN_SWIGLU 1
typedef struct w4a16_chain_op {
  int kind, N, K, splits, x_src, x_shift;
  const void* wq;
  const void* scales;
  const void* zeros;
  const void* x;
  void* y;
} w4a16_chain_op;

/*
 * Host: checks a chain of n_ops GEMVs for M activation rows and writes its
 * plan -- a byte image the caller copies to device memory unchanged -- into
 * `plan` (host memory, plan_bytes bytes; NULL to only ask for sizes).
 * *plan_bytes_needed and *ws_bytes_needed (either may be NULL) receive the
 * plan's size and the workspace size w4a16_chain_run needs. The plan holds
 * the device pointers of `ops`: it is valid as long as those buffers are.
 * Errors: W4A16_EINVAL (a bad kind, shape, split count, pointer, x_src or
 * x_shift, or plan_bytes too small), W4A16_EUNSUPPORTED (M > 8, or K above
 * 32768). Host only; allocates nothing the caller sees.
 */
int w4a16_chain_plan(int M, int n_ops, const w4a16_chain_op* ops, void* plan, size_t plan_bytes,
                     size_t* plan_bytes_needed, size_t* ws_bytes_needed);

/*
 * Runs a chain in one persistent launch on `stream`.
 *   plan_dev: the plan of w4a16_chain_plan, copied to device memory
 *     (16-byte aligned), for the same M.
 *   workspace: device memory of at least the plan's ws_bytes_needed,
 *     16-byte aligned, zero-filled once before its first use. It holds the
 *     launch counter, the error word, the split-K words (left zero by a
 *     completed run) and the tagged outputs the GEMVs hand each other.
 *     One workspace serves every later run of any plan that fits it, on
 *     one stream; runs that may overlap in time need different workspaces.
 *   Every GEMV's y is written. Each output has the arithmetic of the
 *   standalone entry points with the same waves and shares (bit-identical to
 *   w4a16_gemv for K = 3584 unsplit, to w4a16_gemv_swiglu for K = 3584, and
 *   to w4a16_gemv_splitk with 4 splits of K = 18944, given the same input);
 *   every output is within the bound of the plain matrix-vector product.
 * The launch has two workgroups per compute unit and needs all of them
 * resident at once: nothing else may occupy the device's compute units while
 * it runs. The uint32 at byte 8 of the workspace is 0 after a completed run;
 * 1 if a wait ran out (1 s without progress: residency was lost), 2 if the
 * plan does not match M or the workspace. A nonzero word is sticky: later
 * runs return at once until the caller zero-fills the workspace again.
 * Errors (returned): W4A16_EINVAL (NULL or misaligned pointer, ws_bytes
 * below 256), W4A16_EUNSUPPORTED (M other than 1, or the device cannot keep
 * one workgroup per compute unit resident), W4A16_EHIP.
 */
int w4a16_chain_run(int M, const void* plan_dev, void* workspace, size_t ws_bytes, void* stream);

/* Static text for a status code (never NULL). */
const char* w4a16_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
