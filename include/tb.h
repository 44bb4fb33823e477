/*
 * tb.h -- C ABI of the folded-Hadamard ternary Packed-linear library (gfx950).
 *
 * The operation (sources cited by address and section):
 *
 *   [P2] kwkr.cn/news/564617, "ternary weights + folded Hadamard rotation":
 *        every weight matrix was rotated offline in blocks of 1024 along its
 *        input axis by an orthogonal Hadamard transform with an explicit +-1
 *        sign vector (widths 5120 / 6144 / 17408); at run time only the
 *        activation is rotated, by fwht() = normalized transform with scale
 *        1/sqrt(block), signs multiplied before it on the forward pass and
 *        again after it on the inverse pass; the matmul then consumes the
 *        packed 2-bit weights directly (quantized_matmul, transpose=True,
 *        group_size=128, bits=2).
 *   [P2] "packing-format engineering": MLX affine 2-bit container, one fp16
 *        scale and one fp16 bias per group of 128 weights, bias = -scale,
 *        codes {0,1,2} decode to -s/0/s, 2.25 bits/weight.
 *   [P3] lpnh.cn/news/2438023, "text model loading": Packed applies
 *        fwht(x, block, signs) when the module declares a block, then the
 *        quantized matmul on uint32 code words; the embedding module
 *        dequantizes the looked-up row and applies fwht(..., inverse=True).
 *   [P3] "affine 2-bit format and Prism contract v1": block sizes
 *        512/1024/2048/4096, normalized Sylvester-Walsh-Hadamard, axis = the
 *        input (last) dimension, explicit signs, every sign must be +-1.
 *
 * Definitions used by every entry point (K = input width, N = output rows):
 *
 *   codes    uint32 [N][K/16], row-major; code k of a row sits at bits
 *            2*(k%16)..2*(k%16)+1 of word k/16 (little end first).
 *   scales   fp16 bit patterns uint16 [N][K/128]; biases likewise.
 *   W~[n][k] = scales[n][k/128] * c[n][k] + biases[n][k/128],  c = 2-bit code
 *            (code 3 never comes out of tb_pack; kernels decode it affinely).
 *   signs    int8 [K], each +-1; block j of the input uses signs[j*L:(j+1)*L].
 *   R x      = for each block j of L contiguous inputs: H_L (signs .* x) / sqrt(L),
 *            H_L the natural-order Sylvester matrix, H[i][j] = (-1)^popcount(i&j).
 *   Packed linear:  y[b][n] = sum_k W~[n][k] * (R x[b])[k]        (fp32 out)
 *   Embedding:      out[t]  = signs .* (H_L W~[ids[t]]) / sqrt(L) per block
 *   block = 0 means "no rotation": signs must be NULL and R = identity.
 *
 * Conventions:
 *   - Every function returns a status (TB_OK = 0 or a negative TB_ERR_*),
 *     never aborts and never throws; tb_last_error() gives a thread-local
 *     message for the last failure on the calling thread.
 *   - Device entry points take device pointers and a hipStream_t passed as
 *     void* (NULL = the default stream); they only validate scalars and
 *     pointer alignment on the host, never read device memory, never
 *     synchronize, and enqueue asynchronously on the stream.
 *   - The caller owns every buffer.  The library never allocates or frees
 *     memory and keeps no state between calls besides the error string.
 *   - A size of 0 for N, B, rows, T or M is a no-op returning TB_OK; pointers
 *     tied to an empty size may then be NULL.  K must be positive.
 *   - Dimensions are int64; all index arithmetic is 64-bit.
 */
#ifndef TB_H
#define TB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TB_ABI_VERSION 1

/* status codes */
#define TB_OK               0
#define TB_ERR_ARG         -1   /* NULL pointer, negative size, K <= 0, bad flag */
#define TB_ERR_SHAPE       -2   /* K % 128 != 0, K % block != 0, batch out of range */
#define TB_ERR_BLOCK       -3   /* block not in {0, 512, 1024, 2048, 4096} */
#define TB_ERR_UNSUPPORTED -4   /* valid contract value without a kernel */
#define TB_ERR_SIGN        -5   /* a sign other than +-1 (host check) */
#define TB_ERR_CODE        -6   /* ternary value outside {-1,0,1} / code 3 on unpack */
#define TB_ERR_DTYPE       -7   /* activation dtype not TB_F32 / TB_BF16 */
#define TB_ERR_ALIGN       -8   /* pointer not aligned as documented */
#define TB_ERR_HIP         -9   /* the HIP runtime refused a launch */
#define TB_ERR_WORKSPACE  -10   /* workspace NULL or smaller than required */

/* activation dtypes */
#define TB_F32  0
#define TB_BF16 1

/* largest batch the GEMV path takes (prefill batches use tb_ternary_gemm) */
#define TB_GEMV_MAX_BATCH 8

int tb_abi_version(void);
const char* tb_last_error(void);
const char* tb_status_str(int status);

/* ---------------------------------------------------------------------------
 * Host container functions (host pointers; no GPU involved).
 * [P2 "packing-format engineering"]: code = t + 1 ([P1] trdm.cn/news/822023
 * section 3.2 maps -1/0/1 to 0/1/2), 16 codes per uint32 word, bias = -scale
 * (fp16 sign-bit flip, exact); an independent unpack() verifies packing.
 * ------------------------------------------------------------------------ */

/* Pack t (int8 [N][K], values -1/0/1) and scales (fp16 [N][K/128]) into
 * codes (uint32 [N][K/16]), scales_out (copy) and biases_out (= -scales).
 * K % 128 == 0.  Returns TB_ERR_CODE if any t is outside {-1,0,1}; outputs
 * are then unspecified. */
int tb_pack(const int8_t* t, const uint16_t* scales, int64_t N, int64_t K,
            uint32_t* codes, uint16_t* scales_out, uint16_t* biases_out);

/* Unpack codes (uint32 [N][K/16]) to t_out (int8 [N][K]) = code - 1.
 * Returns TB_ERR_CODE if any code is 3 (t_out contents then unspecified). */
int tb_unpack(const uint32_t* codes, int64_t N, int64_t K, int8_t* t_out);

/* Load-time sign check [P3 "affine 2-bit format and Prism contract v1"]:
 * TB_ERR_SIGN unless every signs[k] is +1 or -1.  The device entry points do
 * not re-check signs; a value other than +-1 is used as a multiplier. */
int tb_signs_validate(const int8_t* signs, int64_t K);

/* ---------------------------------------------------------------------------
 * Device entry points (device pointers, asynchronous on `stream`).
 * ------------------------------------------------------------------------ */

/* Device-side pack of the same container as tb_pack (for containers too large
 * to stage on the host).  t, scales, codes, scales_out, biases_out as in
 * tb_pack but in device memory; codes 16-byte aligned.  A value of t outside
 * {-1,0,1} is stored as code 3 and counted into *bad_count (a device int32
 * the caller zeroes first; required). */
int tb_pack_device(const int8_t* t, const uint16_t* scales, int64_t N, int64_t K,
                   uint32_t* codes, uint16_t* scales_out, uint16_t* biases_out,
                   int32_t* bad_count, void* stream);

/* Signed block transform of `rows` rows of K inputs [P3 "text model
 * loading", P2 "ternary weights + folded Hadamard rotation"]:
 *   inverse = 0:  y = H (signs .* x) / sqrt(block)      (forward)
 *   inverse = 1:  y = signs .* (H x) / sqrt(block)      (inverse)
 * x: rows x K of x_dtype (TB_F32 or TB_BF16), row-major; y: rows x K fp32.
 * y may alias x when x is fp32.  block in {512,1024,2048,4096}, K % block == 0.
 * x and y 4-byte aligned (x 2-byte for bf16).
 * Applied forward to the rows of a dense N x K weight matrix W it performs
 * the offline fold W R^T [P2 "ternary weights + folded Hadamard rotation"]:
 * row n of W R^T is the forward transform of row n of W. */
int tb_fwht_signed(const void* x, int x_dtype, float* y, const int8_t* signs,
                   int64_t rows, int64_t K, int block, int inverse, void* stream);

/* Workspace bytes tb_ternary_gemv / _prepare / _run need for batch B and
 * input width K (0 for invalid B or K). */
size_t tb_ternary_gemv_workspace_size(int64_t B, int64_t K);

/* Workspace bytes that let tb_ternary_gemv take its decode-batch path
 * (2 <= B <= TB_GEMV_MAX_BATCH, block 0, 512 or 1024, K a multiple of 256)
 * for an N x K weight matrix: the partial rows of a K-split stream (which
 * grow with N).  Never less than tb_ternary_gemv_workspace_size(B, K); given
 * less than this, tb_ternary_gemv uses its other batch path. */
size_t tb_ternary_gemv_workspace_size_n(int64_t B, int64_t K, int64_t N);

/* Packed linear for decode batches [P3 "text model loading"]:
 *   y[b][n] = sum_k W~[n][k] (R x[b])[k],  b < B <= TB_GEMV_MAX_BATCH.
 * x: B x K (x_dtype), 16-byte aligned; signs 16-byte aligned; codes/scales/
 * biases as defined above (codes 16-byte aligned, scales and biases 4-byte
 * aligned, else TB_ERR_ALIGN); y: B x N fp32 (overwritten, 4-byte aligned).  workspace: device
 * scratch of at least tb_ternary_gemv_workspace_size(B, K) bytes, 16-byte
 * aligned, needing no initialisation; it must not be reused by another call
 * until this one completes on the stream.  Equivalent to
 * tb_ternary_gemv_prepare followed by tb_ternary_gemv_run on one stream.
 * For 2 <= B <= 8, block 0, 512 or 1024 and K a multiple of 256, a
 * workspace of tb_ternary_gemv_workspace_size_n(B, K, N) bytes selects the
 * decode-batch path: each CU transforms one K slice of every batch row into
 * exact integer operands in LDS and streams a 128-row block of the weights
 * over it, and the slices' partial rows are summed in slice order (results
 * do not depend on scheduling). */
int tb_ternary_gemv(const void* x, int x_dtype, int64_t B, int64_t K,
                    const int8_t* signs, int block,
                    const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                    int64_t N, float* y, void* workspace, size_t ws_bytes, void* stream);

/* Bytes of device scratch tb_ternary_gemv_noalloc holds per GPU. */
#define TB_NOALLOC_SCRATCH_BYTES (16u << 20)

/* tb_ternary_gemv for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, result and kernels as tb_ternary_gemv, without the
 * workspace: the library keeps TB_NOALLOC_SCRATCH_BYTES of static device
 * memory per GPU (held until the process ends) and uses it as the workspace.
 * It calls no allocator.  The decode-batch path runs when its partial rows
 * fit there (every N up to 248,320 at K = 5120 and B = 8 does); otherwise
 * the other batch path.  A call whose smallest workspace,
 * tb_ternary_gemv_workspace_size(B, K), exceeds the scratch returns
 * TB_ERR_WORKSPACE before enqueuing anything; TB_ERR_HIP if the scratch's
 * device address cannot be obtained.  Every call on one GPU shares that
 * GPU's scratch, and no call needs it cleared: calls that may overlap on
 * one GPU (concurrent streams, threads) race and must be serialized by the
 * caller. */
int tb_ternary_gemv_noalloc(const void* x, int x_dtype, int64_t B, int64_t K,
                            const int8_t* signs, int block,
                            const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                            int64_t N, float* y, void* stream);

/* First half of tb_ternary_gemv: rotate x (R x, signs then the normalized
 * block transform) and store it in the workspace as exact integer limbs in
 * the matmul kernel's operand layout (format private to the library).  One
 * prepared workspace serves any number of tb_ternary_gemv_run calls with the
 * same B and K -- e.g. the modules that read the same activation. */
int tb_ternary_gemv_prepare(const void* x, int x_dtype, int64_t B, int64_t K,
                            const int8_t* signs, int block, void* workspace, size_t ws_bytes,
                            void* stream);

/* Second half of tb_ternary_gemv: stream the packed weights against a
 * workspace filled by tb_ternary_gemv_prepare(B, K) earlier on the stream. */
int tb_ternary_gemv_run(const void* workspace, size_t ws_bytes, int64_t B, int64_t K,
                        const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                        int64_t N, float* y, void* stream);

/* Workspace bytes tb_ternary_gemm / _prepare / _run need for M rows of width K. */
size_t tb_ternary_gemm_workspace_size(int64_t M, int64_t K);

/* Workspace bytes for M x K activations against N output columns that let
 * tb_ternary_gemm / _run balance the last round of output tiles and read
 * the weights contiguously:
 *  - when the 64 x 512 tiles leave the last round of the GPU's compute
 *    units at most half full, those tiles are split into K slices whose
 *    partial tiles (fp32) follow the prepared activation in the workspace
 *    and are added in slice order by a second kernel (deterministic);
 *  - when M spans at least 4 row tiles (M > 192), the run first copies the
 *    codes and scales into one contiguous record per (512-column tile,
 *    group of 128) after those partials (N/512 x K/128 x 17408 bytes,
 *    rounded up) and the matmul reads that copy (same arithmetic).
 * At least tb_ternary_gemm_workspace_size(M, K); a run with a workspace
 * smaller than this value (but at least that size) computes every tile
 * whole from the weights as stored instead.  Returns
 * tb_ternary_gemm_workspace_size(M, K) for invalid N. */
size_t tb_ternary_gemm_workspace_size_n(int64_t M, int64_t K, int64_t N);

/* Packed linear for prefill (any M >= 1), same definition as the GEMV:
 *   y[m][n] = sum_k W~[n][k] (R x[m])[k]   (fp32 out, M x N)
 * Runs on the block-scaled fp6 x fp4 MFMA: the 2-bit codes are fp4 operands
 * as stored, the rotated activation enters as four signed base-16 fp6 digits
 * per input with one power-of-two exponent per run of 32 inputs (16-bit
 * fixed point relative to the run's largest magnitude); products accumulate
 * in fp32 and the per-group scale and bias are applied in fp32.  Same
 * argument rules as tb_ternary_gemv; equivalent to tb_ternary_gemm_prepare
 * then tb_ternary_gemm_run. */
int tb_ternary_gemm(const void* x, int x_dtype, int64_t M, int64_t K,
                    const int8_t* signs, int block,
                    const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                    int64_t N, float* y, void* workspace, size_t ws_bytes, void* stream);

/* Rotate the M x K activation into the workspace (fp6 digit records, scaled
 * fp16 hi/lo group sums; format private to the library). */
int tb_ternary_gemm_prepare(const void* x, int x_dtype, int64_t M, int64_t K,
                            const int8_t* signs, int block, void* workspace, size_t ws_bytes,
                            void* stream);

/* Multiply a prepared workspace (same M, K) by a packed weight matrix. */
int tb_ternary_gemm_run(const void* workspace, size_t ws_bytes, int64_t M, int64_t K,
                        const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                        int64_t N, float* y, void* stream);

/* ---------------------------------------------------------------------------
 * Multi-module decode [P3 "text model loading": every packed module of the
 * model applies fwht(x, block, signs) and the quantized matmul; a decode step
 * runs all of them].  Many batch-1 Packed linears in two launches: one
 * transforms every module's input, one persistent kernel streams every
 * module's weights.  Each module is the single-row case of tb_ternary_gemv:
 *   y_i[n] = sum_k W~_i[n][k] (R_i x_i)[k]
 * ------------------------------------------------------------------------ */

/* One module (all pointers are device pointers).  x: K activations of the
 * call's x_dtype, 16-byte aligned; signs: K int8 (+-1), 4-byte aligned, or
 * NULL when block = 0; codes: N x K/16 uint32, 16-byte aligned; scales,
 * biases: N x K/128 fp16 bits, 4-byte aligned; y: N fp32, overwritten.
 * K % 256 == 0 and K % block == 0; N may be 0 (the module is skipped). */
typedef struct tb_gemv_module {
  const void* x;
  const int8_t* signs;
  const uint32_t* codes;
  const uint16_t* scales;
  const uint16_t* biases;
  float* y;
  int64_t N;
  int64_t K;
} tb_gemv_module;

/* Bytes of the plan for this module list on the current device (0 for an
 * empty list). */
size_t tb_gemv_multi_plan_size(const tb_gemv_module* mods, int64_t count);

/* Build the plan (host memory, plan_bytes >= tb_gemv_multi_plan_size) for the
 * modules (host array), all sharing x_dtype and block (0, 512 or 1024), and
 * report the workspace the run needs.  Modules with the same x, signs and K
 * (e.g. q/k/v_proj reading one hidden state) share one transform and one
 * operand image.  The plan holds the module table, the
 * transform tasks and a split of all modules' 16-row output tiles into
 * pieces of one module each (shrinking toward the end of the list) that the
 * streaming workgroups take in order from a counter in the workspace; it
 * embeds the device pointers of the modules, so it stays valid while those
 * buffers do.  Errors:
 * TB_ERR_ARG, TB_ERR_SHAPE (K % 256 or K % block), TB_ERR_BLOCK /
 * TB_ERR_UNSUPPORTED (block 2048/4096, or K too large for the kernel's LDS),
 * TB_ERR_DTYPE, TB_ERR_ALIGN, TB_ERR_WORKSPACE (plan buffer too small). */
int tb_gemv_multi_plan(const tb_gemv_module* mods, int64_t count, int x_dtype, int block,
                       void* plan, size_t plan_bytes, size_t* workspace_bytes);

/* tb_gemv_multi_plan on PQ2_0 blocks (the block container below) [P2
 * "packing-format engineering": the same weights as 34-byte GGUF blocks,
 * 2.125 bits/weight, consumed as stored]: each module's codes pointer holds
 * its (N, K/128 * 34) byte array of PQ2_0 blocks (4-byte aligned), and its
 * scales and biases pointers must be NULL (each block carries its scale;
 * bias = -scale).  Same plan size (tb_gemv_multi_plan_size), workspace and
 * run (tb_ternary_gemv_multi); the errors of tb_gemv_multi_plan, with
 * TB_ERR_ARG also for non-NULL scales or biases. */
int tb_pq2_gemv_multi_plan(const tb_gemv_module* mods, int64_t count, int x_dtype, int block,
                           void* plan, size_t plan_bytes, size_t* workspace_bytes);

/* The same on PTQ1_0 blocks [P2 "packing-format engineering": dense trits,
 * 28 bytes per 128 weights, 1.75 bits/weight]: each module's codes pointer
 * holds its (N, K/128 * 28) byte array of PTQ1_0 blocks (4-byte aligned);
 * scales and biases NULL.  Trit bytes above 242 decode to unspecified codes
 * (tb_ptq1_unpack rejects them). */
int tb_ptq1_gemv_multi_plan(const tb_gemv_module* mods, int64_t count, int x_dtype, int block,
                            void* plan, size_t plan_bytes, size_t* workspace_bytes);

/* Run a plan: plan_host is the buffer tb_gemv_multi_plan filled (read on the
 * host for the launch sizes), plan_device a copy of it in device memory
 * (16-byte aligned, read by the kernels; the caller owns both).  workspace:
 * device scratch of the reported size, 16-byte aligned, needing no
 * initialisation, not shared with a concurrent call.  Enqueues two kernels
 * on the stream; every module's y is overwritten. */
int tb_ternary_gemv_multi(const void* plan_host, const void* plan_device,
                          void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * The block containers [P2 "packing-format engineering": the same ternary
 * weights also ship as GGUF blocks of 128 weights; PQ2_0, one 2-bit slot per
 * trit and an fp16 scale, 34 bytes (2.125 bits/weight), a lossless transcode
 * of the MLX container checked by an independent unpack and a bit-compare of
 * the group scales; PTQ1_0, dense trits, 28 bytes (1.75 bits/weight), which
 * need extra arithmetic to decode].  The pages print neither byte layout;
 * the reading implemented here:
 *   block = fp16 scale d (2 bytes, little-endian), then the codes; no bias
 *           is stored: code c (t = c - 1) decodes to (c - 1) d, the MLX
 *           decode with bias = -scale;
 *   PQ2_0   32 code bytes, code k of the block at bits 2 (k % 4) of byte k/4
 *           (byte for byte the MLX group's eight code words);
 *   PTQ1_0  26 trit bytes, byte i = sum_j c[5 i + j] 3^j over j < 5 (the
 *           first code the lowest digit; at most 242); the last byte holds
 *           codes 125..127 the same way (at most 26).
 * A row of K weights is K/128 consecutive blocks; rows are consecutive.
 * ------------------------------------------------------------------------ */

/* MLX container (host) -> PQ2_0 blocks (host, N * K/128 * 34 bytes).
 * TB_ERR_CODE if a bias is not the negated scale (bit for bit) or a code is
 * 3 -- PQ2_0 cannot hold them; blocks are then unspecified. */
int tb_pq2_from_mlx(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                    int64_t N, int64_t K, uint8_t* blocks);

/* PQ2_0 blocks (host) -> MLX container (host): codes, scales = d,
 * biases = -d.  TB_ERR_CODE if a code is 3. */
int tb_pq2_to_mlx(const uint8_t* blocks, int64_t N, int64_t K,
                  uint32_t* codes, uint16_t* scales, uint16_t* biases);

/* Ternary t (int8 [N][K], -1/0/1) and fp16 scales [N][K/128] (host) ->
 * PTQ1_0 blocks (host, N * K/128 * 28 bytes).  TB_ERR_CODE for a t outside
 * {-1,0,1}. */
int tb_ptq1_pack(const int8_t* t, const uint16_t* scales, int64_t N, int64_t K, uint8_t* blocks);

/* PTQ1_0 blocks (host) -> t (int8 [N][K]) and scales (host).  TB_ERR_CODE
 * if a trit byte is out of range (over 242, or over 26 for a last byte). */
int tb_ptq1_unpack(const uint8_t* blocks, int64_t N, int64_t K, int8_t* t, uint16_t* scales);

/* Packed linear on PQ2_0 / PTQ1_0 blocks at batch 1 [P3 "text model
 * loading", with the block decode above]:  y[n] = sum_k W~[n][k] (R x)[k].
 * x: K activations (x_dtype), 16-byte aligned; signs as for tb_ternary_gemv
 * (16-byte aligned); blocks: device, N rows of K/128 blocks, 4-byte aligned
 * (trit bytes are not checked on the device: validate with the host
 * unpack); y: N fp32 (overwritten).  B must be 1 (0 is a no-op; larger
 * batches return TB_ERR_UNSUPPORTED), K a multiple of 256 whose operand
 * image (4.6 KB per 1024 inputs) fits the kernel's LDS beside the band's
 * partial sums -- every K up to 27648 does, TB_ERR_UNSUPPORTED when it does
 * not -- and block 0, 512 or 1024
 * (2048/4096: TB_ERR_UNSUPPORTED).  One launch, no workspace: each
 * workgroup rotates x into its LDS and streams a band of rows. */
int tb_pq2_gemv(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs, int block,
                const uint8_t* blocks, int64_t N, float* y, void* stream);
int tb_ptq1_gemv(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs, int block,
                 const uint8_t* blocks, int64_t N, float* y, void* stream);

/* Embedding lookup with the inverse transform [P3 "text model loading"]:
 *   out[t] = signs .* (H_L W~[ids[t]]) / sqrt(L)   blockwise  (block > 0)
 *   out[t] = W~[ids[t]]                                      (block = 0)
 * ids: int32 [T] (device); table codes/scales/biases of V rows and width K;
 * out: T x K fp32.  An id outside [0, V) yields a row of NaN (no error is
 * returned: ids are not read on the host). */
int tb_embed_inverse(const int32_t* ids, int64_t T,
                     const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                     int64_t V, int64_t K, const int8_t* signs, int block,
                     float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TB_H */
