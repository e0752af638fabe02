/*
 * awq.h - C ABI of the W4A16 weight-only quantized linear layer for MI355X (gfx950).
 *
 * The layer computes y = X' . deq(Wq)^T where
 *   - W[N, K] (row n = output channel) is stored as 4-bit codes q with one binary16
 *     scale s and one 4-bit zero point z per group of `group` consecutive input
 *     channels, deq(q) = (q - z) * s  ("The Ultimate Guide to Quantized LLMs: GPTQ",
 *     section "Understanding Quantized Model Compression": per-block scaling factors
 *     and zero points);
 *   - a per-input-channel scale s_c has been folded into W before quantization,
 *     W' = W diag(s_c), and X' = X diag(s_c)^-1 is applied to the activations
 *     ("Quantization Paradigms for Edge Inference", section 3 "The Math Behind
 *     Activation-Aware Protection (AWQ)", first equation);
 *   - decode (a handful of activation rows) is served by a matrix-vector kernel and
 *     batched decode / prefill by a matrix-core kernel (edgesiliconlab ?p=2015,
 *     section "GEMM vs. GEMV Kernels and Batch Size Dynamics").
 *
 * Conventions shared by every entry point
 *   - Element types: binary16 values travel as uint16_t bit patterns; packed 4-bit
 *     words as int32_t (two's-complement view of the uint32 word).
 *   - Canonical layouts (row-major, all contiguous):
 *       qweight [N][K/8]   int32, element k of row n in bits 4*(k%8).. of word k/8
 *       scales  [K/G][N]   binary16
 *       qzeros  [K/G][N/8] int32, zero of column n in bits 4*(n%8).. of word n/8
 *                          (asymmetric format only; NULL for the symmetric format)
 *       X [M][K], y [M][N] binary16
 *   - Formats: AWQ_FMT_ASYM (scale + zero point), AWQ_FMT_SYM8 (zero fixed at 8).
 *   - Shapes: N % 8 == 0, K % group == 0 (AWQ_ERR_INVALID_ARG otherwise); group 32,
 *     64, or a multiple of 128 (per-channel: group == K), K % 128 == 0, N*K < 2^31,
 *     K <= 2^22, M*K < 2^32 and M*N < 2^32 (AWQ_ERR_UNSUPPORTED otherwise). The pages
 *     fix no group size ("group-wise", "blockwise"); 128 is the tuned case.
 *   - Pointers marked "device" must be device (HBM) addresses on the current HIP
 *     device, 16-byte aligned (AWQ_ERR_MISALIGNED otherwise). The library never
 *     allocates, frees or retains a pointer: the caller owns every buffer.
 *   - Every device entry point is asynchronous and ordered on `stream` (0 = the
 *     null stream). All argument checks run before any launch; a rejected call
 *     launches nothing. A launch failure returns AWQ_ERR_HIP; faults inside a
 *     kernel surface at the caller's next synchronisation, as for any HIP kernel.
 *   - The library holds no mutable global state; calls on different streams that
 *     share no output or workspace buffer may run concurrently.
 */
#ifndef AWQ_H_
#define AWQ_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define AWQ_OK 0
#define AWQ_ERR_INVALID_ARG 1 /* NULL where a buffer is required, negative or
                                 non-divisible size, unknown enum value        */
#define AWQ_ERR_UNSUPPORTED 2 /* valid request the kernels are not built for   */
#define AWQ_ERR_MISALIGNED 3  /* a device pointer is not 16-byte aligned       */
#define AWQ_ERR_WORKSPACE 4   /* packed or workspace buffer smaller than needed */
#define AWQ_ERR_HIP 5         /* the HIP runtime rejected a launch             */

#define AWQ_FMT_ASYM 0
#define AWQ_FMT_SYM8 1

#define AWQ_LAYOUT_CANONICAL 0
#define AWQ_LAYOUT_GFX950 1

/* Static text for a status code (never NULL). */
const char* awq_status_string(int status);

/* Version of the gfx950 packed layout produced by awq_repack. */
int awq_layout_version(void);

/*
 * awq_channel_scale - per-input-channel scale from calibration activations.
 * "Quantization Paradigms for Edge Inference", section 3: salient channels are found
 * from activation magnitudes over a calibration set; the scale is a power of that
 * magnitude.
 *   m_k        = (sum over r < rows of |x_cal[r][k]|) / rows     (float64)
 *   s_c[k]     = binary16(m_k ^ alpha), or 1.0 where m_k == 0
 *   inv_s_c[k] = binary16(1 / s_c[k])
 * x_cal   device, [rows][K] binary16, read only. 1 <= rows <= 8192.
 * s_c     device, [K] binary16, written.
 * inv_s_c device, [K] binary16, written; may be NULL.
 * alpha   exponent in [0, 1]. alpha == 0.5 gives the correctly rounded square root;
 *         other values go through the device pow().
 * Errors: INVALID_ARG (NULL x_cal/s_c, rows or K out of range, alpha outside [0,1]
 *         or NaN), MISALIGNED, HIP.
 */
int awq_channel_scale(const uint16_t* x_cal, int64_t rows, int64_t K, double alpha,
                      uint16_t* s_c, uint16_t* inv_s_c, hipStream_t stream);

/*
 * awq_pack - fold the channel scale into W, quantize each group to 4 bits by
 * round-to-nearest and pack (edgesiliconlab ?p=2015, section "What Is the Core
 * Difference Between AWQ and GPTQ Quantization?": the scaled matrix is quantized
 * with plain round-to-nearest; section "Kernel Execution: Marlin vs. ExLlamaV2 INT4
 * GEMM Micro-Architecture", item 3: 4-bit values packed side by side in a word).
 * For each output row n and group g (v = the group's folded weights
 * binary16(W[n][k] * s_c[k]); rint = round half to even):
 *   AWQ_FMT_ASYM: lo = min(min v, 0), hi = max(max v, 0)
 *                 s = max(binary16((hi - lo) / 15), 2^-24)
 *                 z = clamp(rint(-lo / s), 0, 15)
 *   AWQ_FMT_SYM8: s = max(binary16(max|v| / 7), 2^-24), z = 8
 *   q = clamp(rint(v / s) + z, 0, 15)
 * w       device, [N][K] binary16, read only.
 * s_c     device, [K] binary16 channel scale; NULL means s_c = 1 (plain RTN).
 * qweight device, [N][K/8] int32, written (canonical layout above).
 * scales  device, [K/group][N] binary16, written.
 * qzeros  device, [K/group][N/8] int32, written for ASYM; must be NULL for SYM8.
 * Inputs must be finite and the fold must not overflow binary16.
 * Errors: INVALID_ARG, UNSUPPORTED (group), MISALIGNED, HIP.
 */
int awq_pack(const uint16_t* w, const uint16_t* s_c, int64_t N, int64_t K, int32_t group,
             int32_t fmt, int32_t* qweight, uint16_t* scales, int32_t* qzeros,
             hipStream_t stream);

/* Bytes of the gfx950 packed buffer for an N x K layer (0 if the shape is invalid). */
size_t awq_repacked_bytes(int64_t N, int64_t K, int32_t group, int32_t fmt);

/*
 * awq_repack - canonical (qweight, scales, qzeros) to the gfx950 packed layout that
 * awq_gemv, awq_gemm and awq_dequant(AWQ_LAYOUT_GFX950) read (edgesiliconlab ?p=2015,
 * section "Kernel Execution: Marlin vs. ExLlamaV2 INT4 GEMM Micro-Architecture", item 3:
 * the 4-bit values are laid out so that a shift and a mask recover them in registers
 * right before the matrix instruction; the scales and zero points travel with their
 * block, "The Ultimate Guide to Quantized LLMs: GPTQ", section "Understanding Quantized
 * Model Compression"). A pure integer permutation: no value changes. The layout (version awq_layout_version() == 3):
 *   rows padded to Np = 16 * ceil(N / 16) (padding rows: codes 0, scale 0, zero 0);
 *   codes  at offset 0: unit (t, g) for t < Np/16, g < K/128 at ((t * K/128) + g) * 1024;
 *          in a unit, lane l (0..63) owns bytes [16 l, 16 l + 16): row n = 16 t + l % 16,
 *          four words, word i holding channel k = 128 g + 32 (l / 16) + 8 i + e, e < 8,
 *          at nibble position (e >> 1) + 4 * (e & 1);
 *   sets   each unit carries S = max(1, 128 / group) sets of 16 scales and zeros: set j
 *          of unit g holds canonical group 128 g / group + j for group < 128 (lane l
 *          uses set (l / 16) * S / 4), canonical group 128 g / group for group >= 128;
 *   scales at offset Np * K / 2: binary16 [((t * K/128 + g) * S + j) * 16 + row % 16];
 *   zeros  (ASYM) at the next 256-byte boundary: nibble (r % 8) of 32-bit word
 *          ((t * K/128 + g) * S + j) * 2 + r / 8 for row r = row % 16 of set j.
 * One 128-bit load per lane of a wavefront reads a whole unit; a lane's word i is the
 * B operand of step i of v_mfma_f32_16x16x32_f16 for its row.
 * qweight, scales: device, read only. qzeros: device for ASYM, NULL for SYM8.
 * packed: device, at least awq_repacked_bytes() bytes, written.
 * Errors: INVALID_ARG, UNSUPPORTED, MISALIGNED, WORKSPACE (packed_bytes too small), HIP.
 */
int awq_repack(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
               int64_t N, int64_t K, int32_t group, int32_t fmt, void* packed,
               size_t packed_bytes, hipStream_t stream);

/*
 * awq_dequant - W_d[n][k] = binary16((q - z) * s), one rounding, bit-exact: the
 * dequantization of one block with its scaling factor and zero point ("The Ultimate
 * Guide to Quantized LLMs: GPTQ", section "Understanding Quantized Model Compression").
 * Used as the parity probe of both layouts and as the unfused baseline's first step.
 * layout AWQ_LAYOUT_CANONICAL: w = qweight, with scales and qzeros (NULL for SYM8).
 * layout AWQ_LAYOUT_GFX950:    w = packed buffer; scales and qzeros must be NULL.
 * w_out  device, [N][K] binary16, written.
 * Errors: INVALID_ARG, UNSUPPORTED, MISALIGNED, HIP.
 */
int awq_dequant(const void* w, const uint16_t* scales, const int32_t* qzeros,
                int32_t layout, int64_t N, int64_t K, int32_t group, int32_t fmt,
                uint16_t* w_out, hipStream_t stream);

/*
 * Workspace bytes for an M x N x K call of awq_gemv / awq_gemm (0: none used). The pages
 * define no workspace: it is this library's scratch for splitting K across workgroups
 * and for the once-per-call X' of the prefill kernel. `group` is the layer's group size
 * (the same shape checks as the product entry points; 0 for a shape they reject).
 * awq_gemv keeps every partial sum inside a workgroup and uses none. awq_gemm uses it
 *  - at small M (up to 64 rows, when the call does not run the awq_gemv kernel, see
 *    awq_gemm), when the output has fewer than 80 blocks of its tiling: K is split
 *    across up to four workgroups per block (and in two inside each), the float32 partial
 *    sums [splits][M][N] go to the workspace and a second kernel adds them in split
 *    order (with more blocks K is split only inside the workgroup: no workspace);
 *  - at 65 <= M < 256 when the output blocks alone would leave CUs idle: the same, with
 *    up to eight workgroups per block;
 *  - at M >= 256 with inv_s_c given: X' = binary16(X * inv_s_c) is formed once into the
 *    workspace ([M][K] binary16) and the wide-tile kernel streams it into LDS;
 *  - at M >= 256 when the 128 x 256 output blocks cover fewer than half of the CUs: K is
 *    also split across workgroups, with the float32 partial sums [splits][M][N] placed
 *    after X' (at the next 256-byte boundary) and added in split order.
 * Every call that uses the workspace overwrites the part it uses, so it needs no
 * initialisation; calls that share one workspace must be ordered (same stream). With a
 * NULL workspace awq_gemm runs unsplit and scales X' inside the kernel: same accuracy,
 * slower.
 */
size_t awq_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group);

/*
 * awq_gemv - decode product for 1 <= M <= 16 activation rows (edgesiliconlab ?p=2015,
 * sections "The Mathematics of Memory Bandwidth Saturation" and "GEMM vs. GEMV
 * Kernels and Batch Size Dynamics": at batch 1 the product streams every weight once
 * and is bound by memory bandwidth).
 *   y[m][n] = binary16( sum_k X'[m][k] * (q[n][k] - z[g][n]) * s[g][n] ),
 *   X'[m][k] = binary16(x[m][k] * inv_s_c[k]) (or x itself when inv_s_c is NULL),
 * accumulated in float32. Result within 2e-3 of the exact product of the
 * dequantized weights, relative to max|y|.
 * x       device, [M][K] binary16.   inv_s_c device, [K] binary16, or NULL.
 * packed  device, gfx950 layout from awq_repack for (N, K, group, fmt).
 * y       device, [M][N] binary16, written.
 * ws      device workspace of ws_bytes >= awq_workspace_bytes() bytes, or NULL with
 *         ws_bytes == 0.
 * M == 0 returns AWQ_OK without launching. Deterministic: the same inputs give the
 * same bits on every call.
 * Errors: INVALID_ARG, UNSUPPORTED (M > 16, group), MISALIGNED, WORKSPACE, HIP.
 */
int awq_gemv(const uint16_t* x, const uint16_t* inv_s_c, const void* packed, int64_t M,
             int64_t N, int64_t K, int32_t group, int32_t fmt, uint16_t* y, void* ws,
             size_t ws_bytes, hipStream_t stream);

/*
 * awq_gemm - batched-decode / prefill product for any M >= 1 on the matrix cores
 * (edgesiliconlab ?p=2015, "GEMM vs. GEMV Kernels and Batch Size Dynamics": larger
 * batches turn the product into a matrix-matrix multiply; section "Kernel Execution:
 * Marlin vs. ExLlamaV2 INT4 GEMM Micro-Architecture": weights are unpacked to
 * binary16 just before the matrix instruction). Same arguments, math and accuracy as
 * awq_gemv; the dequantized weights fed to the matrix cores are exactly W_d. It runs
 * the awq_gemv kernel instead where that is faster (no split of K, no second launch):
 * at M <= 2; at M <= 4 when ceil(N / 16) * K / 128 <= 32768; and up to 16 rows when
 * ceil(N / 16) <= 256 and M * K / 128 <= 704. Which
 * kernel runs and the split of K (see awq_workspace_bytes) depend only on M, N, K and
 * whether a large enough workspace is given, so repeated calls give the same bits.
 * Errors: INVALID_ARG, UNSUPPORTED, MISALIGNED, WORKSPACE, HIP.
 */
int awq_gemm(const uint16_t* x, const uint16_t* inv_s_c, const void* packed, int64_t M,
             int64_t N, int64_t K, int32_t group, int32_t fmt, uint16_t* y, void* ws,
             size_t ws_bytes, hipStream_t stream);

/*
 * awq_gemm_noalloc - awq_gemm for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, checks, kernels and results as awq_gemm given a workspace of
 * awq_workspace_bytes(M, N, K, group) bytes (the same bits), without the workspace
 * arguments: the library uses a device array of its own, 64 MiB per GPU, which each GPU
 * the library runs on holds until the process ends (its address is looked up once per
 * device on the first call there). The call allocates and frees nothing.
 * Calls whose awq_workspace_bytes exceeds 64 MiB return AWQ_ERR_WORKSPACE before any
 * launch (use awq_gemm with a caller workspace for those, e.g. M = 4096 on K = 28672).
 * Every call on one GPU shares that GPU's array and overwrites the part it uses (nothing
 * in it has to start at zero): calls that overlap on one GPU (different streams, or
 * host threads without ordering) race and must not be issued.
 * Errors: INVALID_ARG, UNSUPPORTED, MISALIGNED, WORKSPACE, HIP.
 */
int awq_gemm_noalloc(const uint16_t* x, const uint16_t* inv_s_c, const void* packed, int64_t M,
                     int64_t N, int64_t K, int32_t group, int32_t fmt, uint16_t* y,
                     hipStream_t stream);

/*
 * Decode chain: the M = 1 products of one decoder block in a single launch
 * (edgesiliconlab ?p=2015, section "The Mathematics of Memory Bandwidth Saturation":
 * at batch 1 a token costs the bytes of every weight it streams, so the time between
 * products is lost bandwidth). Each layer i computes, as awq_gemv does at M = 1,
 *   y_i[n] = binary16( sum_k X'_i[k] * (q_i[n][k] - z) * s ),  X'_i = binary16(in_i * inv_s_c_i),
 * where in_i is the caller's x when src == -1 and layer src's output y_src otherwise
 * (src < i: the layer starts once every output of layer src is written). Layers that
 * do not depend on each other overlap; the weights of a layer are read while the
 * layers before it finish. Within 2e-3 of the exact product of the dequantized
 * weights with the layer's binary16 input, relative to max|y_i|; the same bits on
 * every call.
 */
typedef struct awq_chain_layer {
  const uint16_t* x;       /* device, [K] binary16; used when src == -1, else ignored */
  const uint16_t* inv_s_c; /* device, [K] binary16, or NULL                         */
  const void* packed;      /* device, gfx950 layout from awq_repack for (N, K, group, fmt) */
  uint16_t* y;             /* device, [N] binary16, written                          */
  int64_t N, K;
  int32_t group, fmt;
  int32_t src;             /* -1, or the index of an earlier layer whose N equals K  */
  int32_t reserved;        /* set to 0                                               */
} awq_chain_layer;

/* Most layers one awq_gemv_chain call takes. */
#define AWQ_CHAIN_MAX_LAYERS 8

/*
 * Bytes of the chain state buffer. The caller allocates it (device, 16-byte aligned),
 * sets it to zero once before the first call, and passes the same buffer to every
 * call; each call leaves it as it found it, except word 0 (uint32): bit 0 set means a
 * wait inside a call ran out (about 0.17 s), and that call's outputs are not valid
 * (clear the word, or the whole buffer, before the next call).
 */
size_t awq_chain_state_bytes(void);

/*
 * awq_gemv_chain - run `n_layers` M = 1 products in one launch, in the order given.
 * layers  host array of n_layers descriptors (read during the call only).
 * Shapes: as awq_gemv, and 1920 <= K <= 16384, group a multiple of 128 (per-channel
 * included: AWQ_ERR_UNSUPPORTED otherwise). Each layer's y must be a buffer of its own,
 * not read by any layer as x. n_layers == 0 returns AWQ_OK without launching;
 * n_layers > AWQ_CHAIN_MAX_LAYERS is AWQ_ERR_UNSUPPORTED.
 * state   device, awq_chain_state_bytes() bytes (see above). Calls that share a state
 *         buffer must be ordered (same stream); a call uses every CU of the device and
 *         waits inside the launch for its own earlier layers, so it must not share the
 *         device with a kernel that waits for it.
 * Errors: INVALID_ARG (NULL buffer, src out of range, input length != K),
 *         UNSUPPORTED, MISALIGNED, HIP.
 */
int awq_gemv_chain(const awq_chain_layer* layers, int32_t n_layers, void* state,
                   hipStream_t stream);

/*
 * Workspace bytes awq_scale_search needs for (rows, N, K, group, fmt); 0 for arguments it
 * would reject.
 */
size_t awq_scale_search_workspace_bytes(int64_t rows, int64_t N, int64_t K, int32_t group,
                                        int32_t fmt);

/*
 * awq_scale_search - grid search of the AWQ channel-scale exponent ("Quantization
 * Paradigms for Edge Inference: AWQ, GPTQ, and FP8 Matrix Cores", section 3, second
 * equation: the scale minimises || W X - Q(W diag(s)) diag(s)^-1 X || on calibration
 * data). The pages leave the search space open; it is s = (mean_r |x_cal[r][k]|)^alpha
 * (as awq_channel_scale) for alpha = i / grid, i = 0 .. grid.
 * For each alpha the candidate is built and applied with this library's own kernels,
 * as it would be deployed (awq_channel_scale, awq_pack, awq_repack, awq_gemm on the
 * calibration rows, binary16 output), and scored against X_cal . W^T formed once in
 * float32 from the unquantized binary16 weights:
 *   losses[i] = sqrt( sum_{r,n} (ref[r][n] - y_i[r][n])^2 ),  summed in float64 in a
 *   fixed order (the same bits on every call);
 *   best_alpha[0] = i / grid for the first i with the smallest loss.
 * w       device, [N][K] binary16 (unquantized, unfolded weights).
 * x_cal   device, [rows][K] binary16 calibration activations, 1 <= rows <= 256.
 * losses  device, [grid + 1] float64, written.  best_alpha device, [1] float64, written.
 * ws      device workspace of ws_bytes >= awq_scale_search_workspace_bytes() bytes
 *         (overwritten; holds the candidate's quantized layer and products).
 * 1 <= grid <= 1000. Asynchronous on `stream` like every device entry point: the
 * results are valid after the caller synchronises the stream.
 * Errors: INVALID_ARG, UNSUPPORTED (group, sizes), MISALIGNED (w, x_cal, ws not 16-byte
 * or losses, best_alpha not 8-byte aligned), WORKSPACE, HIP.
 */
int awq_scale_search(const uint16_t* w, const uint16_t* x_cal, int64_t rows, int64_t N,
                     int64_t K, int32_t group, int32_t fmt, int32_t grid, double* losses,
                     double* best_alpha, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_H_ */
