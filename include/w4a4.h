/*
 * w4a4.h -- C ABI of the MI355X (gfx950) W4A4 + INT8-outlier linear layer.
 *
 * The layer is the hybrid scheme of QUIK ("QUIK: Towards End-to-End 4-Bit
 * Inference on Generative Large Language Models", abstract) in the form the
 * Atom summary page gives it ("Atom: Low-bit Quantization for Efficient and
 * Accurate LLM Serving", Summary paragraph 2; Key points item 5; Interesting
 * ideas I1-I3):
 *   - a small set O of outlier input channels is moved to a contiguous tail
 *     (perm = ascending channels not in O, then ascending channels in O) and
 *     kept in INT8;
 *   - every other channel is quantized to INT4, symmetric round-to-nearest
 *     with an absmax scale per row (group == 0) or per group of `group`
 *     consecutive reordered channels;
 *   - activation scales are computed for every input at run time, weights are
 *     quantized once;
 *   - Y = sum_t sa4[m,t] sw4[n,t] acc4_t[m,n] + sa8[m] sw8[n] acc8[m,n], with
 *     exact int32 accumulators and an fp32 epilogue rounded to fp16.
 *
 * Quantizer, for every block v of a row (INT4: qmax = 7, INT8: qmax = 127):
 *   s = fl32(max|v| / qmax);  q = s == 0 ? 0 : clamp(rint(fl32(v / s)),
 *   -qmax-1, qmax), with correctly rounded fp32 division and ties to even.
 *
 * Conventions for every call below
 *   - All matrices are row-major. X is fp16 [M, ldx] (tokens x channels),
 *     W is fp16 [N, ldw] (output channels x channels, torch.nn.Linear layout),
 *     Y is fp16 [M, ldy].
 *   - K_n = K - n_out; G = w4a4_num_groups(K_n, group).
 *   - Packed INT4 operand: uint8 [rows, w4a4_pitch4_bytes(K_n)]; byte i of a
 *     row = (q[2i] & 0xF) | (q[2i+1] & 0xF) << 4 (two's complement nibbles,
 *     low nibble first); bytes past K_n/2 are zero and are part of the
 *     format.
 *   - INT8 tail: int8 [rows, w4a4_pitch8_bytes(n_out)], zero padded.
 *   - INT4 scales: fp32 [rows, G] row-major; INT8 tail scales: fp32 [rows]
 *     (0 when n_out == 0).
 *   - Device pointers are caller-owned device memory; the library allocates
 *     and frees nothing. Device pointers must be 16-byte aligned (fp16 Y:
 *     2-byte aligned); ldx and ldw must be multiples of 8 elements.
 *   - Every device call is asynchronous on `stream` (a hipStream_t; NULL is
 *     the null stream). Host checks run first; on any error nothing is
 *     launched and nothing is written. A launch failure returns
 *     W4A4_ERR_HIP; faults inside a kernel surface at the caller's next
 *     synchronisation.
 *   - M == 0 or N == 0 is a valid empty call and launches nothing.
 *   - Calls are stateless and thread-safe; calls that share output buffers
 *     on different streams race.
 */
#ifndef W4A4_H
#define W4A4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum w4a4_status {
    W4A4_OK = 0,
    W4A4_ERR_INVALID_ARG = 1, /* null pointer, bad size, group not dividing K_n, ld too small,
                                 repeated / out-of-range outlier index                       */
    W4A4_ERR_UNSUPPORTED = 2, /* shape outside the kernels' int32 range guard or a group size
                                 the GPU kernels do not implement                            */
    W4A4_ERR_ALIGNMENT = 3,   /* misaligned pointer or leading dimension                     */
    W4A4_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed                  */
    W4A4_ERR_WORKSPACE = 5    /* workspace smaller than the query function asks for          */
} w4a4_status;

typedef void *w4a4_stream; /* hipStream_t */

/* Human-readable name of a status code (static storage). */
const char *w4a4_status_string(int status);

/* Number of INT4 scale groups per row: K_n / group, 1 when group == 0, 0 when
 * K_n == 0. Returns -1 when group < 0 or group does not divide K_n. */
int32_t w4a4_num_groups(int32_t K_n, int32_t group);

/* Row pitch in bytes of a packed INT4 operand: round_up(K_n, 128) / 2. */
int64_t w4a4_pitch4_bytes(int32_t K_n);

/* Row pitch in bytes of an INT8 tail operand: round_up(n_out, 64). */
int64_t w4a4_pitch8_bytes(int32_t n_out);

/* Host helper: perm[0..K) = ascending channels not in outlier_idx, then the
 * outlier channels ascending (Atom summary page, Interesting ideas I1: the
 * outlier channels become one contiguous block at the end). outlier_idx may
 * be unsorted. Host pointers. INVALID_ARG on a repeated or out-of-range
 * index, K <= 0, or n_out outside [0, K]. The caller copies perm to the
 * device for the calls below. */
w4a4_status w4a4_make_perm(int32_t K, const int32_t *outlier_idx, int32_t n_out,
                           int32_t *perm);

/* Activation producer (Atom summary page, Summary paragraph 2: scales
 * computed for each input at run time; reordering fused into one pass).
 * For every token row m of X: gather by perm, quantize the K_n head to INT4
 * (scale per row or per group) and the n_out tail to INT8, pack.
 *   X    device fp16 [M, ldx]          perm device int32 [K] (a permutation)
 *   Aq4  device uint8 [M, pitch4]      Aq8  device int8 [M, pitch8] (NULL if n_out == 0)
 *   sa4  device fp32 [M, G]            sa8  device fp32 [M] (written 0 if n_out == 0)
 * GPU group sizes: 0 or a multiple of 128 dividing K_n (else UNSUPPORTED).
 * perm is trusted to be a permutation of [0, K); an index outside [0, K) is
 * undefined behaviour. A NULL perm is the identity order (no reordering). */
w4a4_status w4a4_quant_reorder_act(const void *X, int64_t ldx, const int32_t *perm,
                                   int32_t M, int32_t K, int32_t n_out, int32_t group,
                                   void *Aq4, void *Aq8, float *sa4, float *sa8,
                                   w4a4_stream stream);

/* Producer fused with the RMSNorm that precedes the layer (Atom summary page,
 * Summary paragraph 2 and Interesting ideas I2: quantization fused into the
 * operators around the GEMM; the norm is the standard RMSNorm of the Llama
 * models the pages evaluate). Each token row is normalized in registers and
 * quantized as by w4a4_quant_reorder_act; the normalized row never goes to
 * memory. The normalized value of channel c is
 *   y_c = fp16( gamma[c] * fp16( fp32(x_c) * rstd ) )      (both roundings to nearest even)
 *   rstd = fp32( 1 / sqrt( fp64(S) / K + eps ) )            (binary64 operations)
 * with S = sum_c x_c^2 computed exactly (every x_c^2 is a multiple of 2^-48);
 * rstd = 0 when the mean square plus eps is 0 (a zero row with eps = 0).
 *   gamma device fp16 [K], original channel order (2-byte aligned)
 *   eps   >= 0 and finite (else INVALID_ARG)
 *   rstd  device fp32 [M] (may be NULL): the norm factor of each row
 * Other arguments and layouts as w4a4_quant_reorder_act. The normalized row
 * must be finite (|gamma[c]| * sqrt(K) below the fp16 range is enough). */
w4a4_status w4a4_rmsnorm_quant_reorder_act(const void *X, int64_t ldx, const void *gamma, float eps,
                                           const int32_t *perm, int32_t M, int32_t K, int32_t n_out,
                                           int32_t group, void *Aq4, void *Aq8, float *sa4,
                                           float *sa8, float *rstd, w4a4_stream stream);

/* Offline weight preparation (QUIK abstract: outlier weights kept in higher
 * precision; Atom summary page: INT4 weights, 8-bit outlier channels in the
 * same reordered layout). The same quantizer applied to the N rows of W, with
 * the same perm as the activations (outliers are input channels).
 *   W    device fp16 [N, ldw]   Wq4 device uint8 [N, pitch4]   Wq8 device int8 [N, pitch8]
 *   sw4  device fp32 [N, G]     sw8 device fp32 [N]
 * Same argument rules as w4a4_quant_reorder_act. */
w4a4_status w4a4_pack_int4_weights(const void *W, int64_t ldw, const int32_t *perm,
                                   int32_t N, int32_t K, int32_t n_out, int32_t group,
                                   void *Wq4, void *Wq8, float *sw4, float *sw8,
                                   w4a4_stream stream);

/* Bytes of device workspace w4a4_outlier_gemm needs for this shape (0 means
 * none; a NULL workspace is then allowed). Shapes with few output tiles for
 * the chip (decode batches) split K across workgroups; the workspace then
 * holds one arrival counter per output tile (a fixed 2048-byte block at its
 * start, the same place for every shape) and fp32 partial sums
 * [splits, M, N]. A pure function of the shape. */
size_t w4a4_outlier_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t n_out,
                                         int32_t group);

/* Name of the GPU kernel w4a4_outlier_gemm launches for this shape, as a
 * kernel trace prints it (the template arguments the shape fixes included;
 * for the 256 x 256 tile kernel, whose edge instantiation also depends on Y,
 * the name without them), for profiling and benchmarks: a static string owned
 * by the library, or NULL for a shape the call would reject. A pure function
 * of the shape, like the workspace size. */
const char *w4a4_outlier_gemm_kernel_name(int32_t M, int32_t N, int32_t K, int32_t n_out,
                                          int32_t group);

/* Mixed-precision GEMM (Atom summary page, Summary paragraph 2 and
 * Interesting ideas I3; Key points item 5 for the symmetric epilogue):
 * INT4 x INT4 over the K_n head plus INT8 x INT8 over the outlier tail, int32
 * accumulation, fp32 scale epilogue, fp16 output
 *   Y[m, n] = fp16( sum_t sa4[m,t] sw4[n,t] acc4_t[m,n] + sa8[m] sw8[n] acc8[m,n] ).
 * Operands in the layouts above (from the two calls above). Y device fp16
 * [M, ldy], ldy >= N. GPU constraints (UNSUPPORTED otherwise): K_n * 16384 <
 * 2^31 and n_out * 16384 < 2^31 (int32 range of the widened accumulators);
 * max(M, N) * max(pitch4, pitch8) < 2^32 (32-bit row offsets); group 0 or a
 * multiple of 128 (the pages fix no group size; one GPU K-tile of 128 INT4
 * channels then never straddles two groups, and the workloads use 0 and 128).
 * workspace: device memory of at least w4a4_outlier_gemm_workspace_bytes
 * bytes, 256-byte aligned (ALIGNMENT otherwise; WORKSPACE if too small). It
 * must be all zero before the first call that uses it (allocate it zeroed
 * once); every call leaves its counters at zero again when it completes, so
 * it can be reused by later calls of any shape. Calls that share a workspace
 * must not run concurrently. With split K the partial sums are added in a
 * fixed order, so results are bit-identical from call to call. */
w4a4_status w4a4_outlier_gemm(const void *Aq4, const void *Aq8, const float *sa4,
                              const float *sa8, const void *Wq4, const void *Wq8,
                              const float *sw4, const float *sw8, int32_t M, int32_t N,
                              int32_t K, int32_t n_out, int32_t group, void *Y,
                              int64_t ldy, void *workspace, size_t workspace_bytes,
                              w4a4_stream stream);

/* The same call with the accumulator export (test path): it launches the
 * kernel w4a4_outlier_gemm launches for the shape, with the same main loop,
 * writes the same Y, and also stores the exact integer accumulators
 *   acc4 device int32 [G, M, N] (one slice per scale group; NULL allowed when K_n == 0)
 *   acc8 device int32 [M, N]    (NULL allowed when n_out == 0)
 * (zeroed by the call first: kernels whose waves or workgroups each hold part
 * of a group's sum add their parts). Same arguments and constraints as
 * w4a4_outlier_gemm otherwise. */
w4a4_status w4a4_outlier_gemm_i32(const void *Aq4, const void *Aq8, const float *sa4,
                                  const float *sa8, const void *Wq4, const void *Wq8,
                                  const float *sw4, const float *sw8, int32_t M, int32_t N,
                                  int32_t K, int32_t n_out, int32_t group, void *Y,
                                  int64_t ldy, void *workspace, size_t workspace_bytes,
                                  int32_t *acc4, int32_t *acc8, w4a4_stream stream);

/* Name of the GPU kernel that computes w4a4_quant_gemm's product for this
 * shape (and w4a4_rmsnorm_quant_gemm's when M == 1): "decode_fused_kernel" when the quantizer is fused into it (see
 * w4a4_quant_gemm), else the kernel w4a4_outlier_gemm launches. A static
 * string owned by the library, or NULL for a shape the call would reject. */
const char *w4a4_quant_gemm_kernel_name(int32_t M, int32_t N, int32_t K, int32_t n_out,
                                        int32_t group);

/* Bytes of device workspace w4a4_quant_gemm needs: the GEMM's own workspace
 * first (its 2048-byte arrival-counter block at offset 0, reserved for every
 * shape, so one workspace can serve calls of any shape in turn), then the
 * quantized activations (Aq4, Aq8, sa4, sa8 for M rows). The same
 * zero-on-first-use rule as w4a4_outlier_gemm's workspace. */
size_t w4a4_quant_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t n_out,
                                       int32_t group);

/* The fused layer (Atom summary page, Interesting ideas I2: quantization and
 * reordering run as part of the layer's own launches): w4a4_quant_reorder_act
 * on X into the caller's workspace, then w4a4_outlier_gemm with the
 * pre-packed weights, both on `stream`. Small decode batches (M <= 2,
 * group 128, n_out <= 128, K_n <= 16384) take one launch instead: the GEMM's
 * workgroups gather and quantize the token rows themselves, with the same
 * arithmetic, so Y is bit-identical to the two-launch result; the workspace is
 * then left untouched. */
w4a4_status w4a4_quant_gemm(const void *X, int64_t ldx, const int32_t *perm, const void *Wq4,
                            const void *Wq8, const float *sw4, const float *sw8, int32_t M,
                            int32_t N, int32_t K, int32_t n_out, int32_t group, void *Y,
                            int64_t ldy, void *workspace, size_t workspace_bytes,
                            w4a4_stream stream);

/* w4a4_quant_gemm without a caller workspace, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the workspace is a library-owned device
 * array of w4a4_quant_gemm_static_max_bytes() bytes (32 MiB), one copy per
 * GPU, held until the process ends; the call allocates nothing. Arguments,
 * results and kernels are those of w4a4_quant_gemm; UNSUPPORTED when
 * w4a4_quant_gemm_workspace_bytes for the shape exceeds the array. Every call
 * on a GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams or host threads) race. The array keeps the last call's contents;
 * the split-K arrival counters at its start are cleared by a kernel on
 * `stream` before the launches that use them. */
size_t w4a4_quant_gemm_static_max_bytes(void);
w4a4_status w4a4_quant_gemm_static(const void *X, int64_t ldx, const int32_t *perm, const void *Wq4,
                                   const void *Wq8, const float *sw4, const float *sw8, int32_t M,
                                   int32_t N, int32_t K, int32_t n_out, int32_t group, void *Y,
                                   int64_t ldy, w4a4_stream stream);

/* The fused layer behind an RMSNorm: w4a4_rmsnorm_quant_reorder_act on X
 * into the caller's workspace (the same size as w4a4_quant_gemm's), then
 * w4a4_outlier_gemm, both on `stream`. gamma and eps as in
 * w4a4_rmsnorm_quant_reorder_act. A single decode token (M == 1) in the
 * shapes where w4a4_quant_gemm takes one launch takes one launch here too
 * (norm, quantizer and GEMM in the same workgroups, the same arithmetic, a
 * bit-identical Y). */
w4a4_status w4a4_rmsnorm_quant_gemm(const void *X, int64_t ldx, const void *gamma, float eps,
                                    const int32_t *perm, const void *Wq4, const void *Wq8,
                                    const float *sw4, const float *sw8, int32_t M, int32_t N,
                                    int32_t K, int32_t n_out, int32_t group, void *Y, int64_t ldy,
                                    void *workspace, size_t workspace_bytes, w4a4_stream stream);

/* ---------------------------------------------------------------------------
 * FP6 prefill path. The layer's INT4 x INT4 sums (Atom summary page, Summary
 * paragraph 2 and Key points item 5) formed on CDNA4's FP6 matrix
 * instruction: every INT4 code q is held as the FP6 E2M3 code of q / 8 (sign
 * bit 5, exponent bits 4..3 with bias 1, mantissa bits 2..0, as the OCP
 * Microscaling Formats v1.0 define E2M3; exact for |q| <= 8, and the code is
 * |q| with the sign in bit 5) and multiplied
 * with an operand block scale of 2^3, so products and partial sums are the
 * integers below 2^24 of the codes, and the fp32 accumulators hold the exact integer
 * sums: the results are those of w4a4_outlier_gemm, with the same int32
 * accumulators. The INT8 outlier tail is unchanged.
 *
 * u6 operand of `rows` rows (K_n head channels): rows in blocks of 32
 * (rows past the last are code 0) and channels in tiles of 64 (T = pitch4 /
 * 32 tiles, code 0 past K_n); the block of row block b and tile t is 1536
 * bytes at offset (b * T + t) * 1536. Each row's two 32-channel chunks h = 0,
 * 1 of the tile are 192-bit images holding code i of the chunk at bits 6i ..
 * 6i+5 (little-endian); image bytes 0..15 of row r's chunk h sit at 512 h +
 * 16 r of the block and image bytes 16..23 at 1024 + 256 h + 8 r (the layout
 * the GEMM's LDS reads want, so whole blocks are copied).
 * --------------------------------------------------------------------------- */

/* Bytes of a u6 operand: ceil(rows / 32) * (pitch4 / 32) * 1536 (0 when rows
 * or K_n is 0; -1 for negative sizes). */
int64_t w4a4_u6_bytes(int32_t rows, int32_t K_n);

/* Convert packed INT4 nibbles Q4 device uint8 [rows, pitch4] (the layout of
 * Aq4 / Wq4 above) to a u6 operand U6 device uint8 [w4a4_u6_bytes(rows,
 * K_n)]. Weights are converted once, offline. Both pointers 16-byte aligned
 * (ALIGNMENT). */
w4a4_status w4a4_repack_u6(const void *Q4, int32_t rows, int32_t K_n, void *U6, w4a4_stream stream);

/* The activation producer of the FP6 path (QUIK abstract; Atom summary page,
 * Summary paragraph 2 and Interesting ideas I2): w4a4_quant_reorder_act with
 * the INT4 head written straight into a u6 operand Au6 device uint8
 * [w4a4_u6_bytes(M, K_n)] (rows past M up to the end of their 32-row block
 * are written as code 0) instead of packed nibbles. Codes, scales and the
 * INT8 tail are those of w4a4_quant_reorder_act; Au6 equals w4a4_repack_u6
 * of its Aq4 byte for byte. Group sizes as w4a4_quant_reorder_act; Au6
 * 16-byte aligned; other arguments as w4a4_quant_reorder_act. */
w4a4_status w4a4_quant_reorder_act_u6(const void *X, int64_t ldx, const int32_t *perm, int32_t M,
                                      int32_t K, int32_t n_out, int32_t group, void *Au6, void *Aq8,
                                      float *sa4, float *sa8, w4a4_stream stream);

/* The FP6 path's producer fused with the preceding RMSNorm (Atom summary
 * page, Interesting ideas I2: the quantization fused into the operator in
 * front of the GEMM): w4a4_rmsnorm_quant_reorder_act with the INT4 head
 * written as the u6 operand Au6 (as w4a4_quant_reorder_act_u6 writes it).
 * Codes, scales, rstd and the INT8 tail are those of
 * w4a4_rmsnorm_quant_reorder_act; Au6 equals w4a4_repack_u6 of its Aq4 byte
 * for byte. Arguments as those two calls. */
w4a4_status w4a4_rmsnorm_quant_reorder_act_u6(const void *X, int64_t ldx, const void *gamma, float eps,
                                              const int32_t *perm, int32_t M, int32_t K, int32_t n_out,
                                              int32_t group, void *Au6, void *Aq8, float *sa4,
                                              float *sa8, float *rstd, w4a4_stream stream);

/* Name of the kernel w4a4_outlier_gemm_fp6 launches for this shape (as a
 * kernel trace prints it), or NULL for a shape it rejects. */
const char *w4a4_outlier_gemm_fp6_kernel_name(int32_t M, int32_t N, int32_t K, int32_t n_out,
                                              int32_t group);

/* The mixed-precision GEMM with u6 INT4 operands (Au6 for the M activation
 * rows, Wu6 for the N weight rows); the INT8 tails and the scales as for
 * w4a4_outlier_gemm, and the same Y definition. Constraints: group 0 (one
 * INT4 scale per row) or 128 with K_n a multiple of 128, K_n > 0, at most
 * 256 outlier channels (UNSUPPORTED otherwise), plus those of
 * w4a4_outlier_gemm. No workspace. */
w4a4_status w4a4_outlier_gemm_fp6(const void *Au6, const void *Aq8, const float *sa4,
                                  const float *sa8, const void *Wu6, const void *Wq8,
                                  const float *sw4, const float *sw8, int32_t M, int32_t N,
                                  int32_t K, int32_t n_out, int32_t group, void *Y, int64_t ldy,
                                  w4a4_stream stream);

/* The same call with the accumulator export (test path): the same kernel and
 * main loop, the same Y, and the exact integer sums acc4 device int32 [1, M,
 * N] and acc8 device int32 [M, N] (NULL allowed when n_out == 0). */
w4a4_status w4a4_outlier_gemm_fp6_i32(const void *Au6, const void *Aq8, const float *sa4,
                                      const float *sa8, const void *Wu6, const void *Wq8,
                                      const float *sw4, const float *sw8, int32_t M, int32_t N,
                                      int32_t K, int32_t n_out, int32_t group, void *Y,
                                      int64_t ldy, int32_t *acc4, int32_t *acc8,
                                      w4a4_stream stream);

/* Workspace bytes of w4a4_quant_gemm_fp6 (no contents required on entry). */
size_t w4a4_quant_gemm_fp6_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t n_out,
                                           int32_t group);

/* The fused prefill layer on the FP6 path (Atom summary page, Interesting
 * ideas I2): w4a4_quant_reorder_act_u6 on X and w4a4_outlier_gemm_fp6 with
 * the pre-converted weights Wu6 (w4a4_repack_u6 of Wq4), both on `stream`,
 * with the caller's workspace. The
 * codes, scales and integer sums are those of w4a4_quant_gemm. Constraints of
 * w4a4_outlier_gemm_fp6. */
w4a4_status w4a4_quant_gemm_fp6(const void *X, int64_t ldx, const int32_t *perm, const void *Wu6,
                                const void *Wq8, const float *sw4, const float *sw8, int32_t M,
                                int32_t N, int32_t K, int32_t n_out, int32_t group, void *Y,
                                int64_t ldy, void *workspace, size_t workspace_bytes,
                                w4a4_stream stream);

/* W4A8 GEMM (the QQQ abstract on the "smoothquant" tag page: 4-bit weights with 8-bit activations, a
 * per-channel and a per-group GEMM), without outlier channels:
 *   Y[m, n] = fp16( sa8[m] * sum_t sw4[n, t] * acc_t[m, n] ),
 *   acc_t[m, n] = sum over the channels j of group t of qa8[m, j] * qw4[n, j].
 * Operands, all in the original channel order (a NULL perm):
 *   Aq8 device int8 [M, K], sa8 device fp32 [M]: w4a4_quant_reorder_act(X, ldx,
 *       NULL, M, K, n_out = K, group = 0, NULL, Aq8, NULL, sa8) (per-token INT8)
 *   Wq4 device uint8 [N, K / 2], sw4 device fp32 [N, G]: w4a4_pack_int4_weights(W,
 *       ldw, NULL, N, K, n_out = 0, group, Wq4, NULL, sw4, NULL)
 * G = K / group, or 1 for group 0 (one scale per output channel). Y device
 * fp16 [M, ldy], ldy >= N. UNSUPPORTED unless K is a multiple of 128, group
 * is 0 or a multiple of 128, and K * 16384 < 2^31. INVALID_ARG for a group
 * not dividing K or a NULL pointer; ALIGNMENT unless Aq8 and Wq4 are 16-byte
 * aligned. */
w4a4_status w4a4_w4a8_gemm(const void *Aq8, const float *sa8, const void *Wq4, const float *sw4,
                           int32_t M, int32_t N, int32_t K, int32_t group, void *Y, int64_t ldy,
                           w4a4_stream stream);

/* Accumulator export of the same main loop (test path): acc device int32
 * [G, M, N], the exact integer sums of every scale group. */
w4a4_status w4a4_w4a8_gemm_i32(const void *Aq8, const void *Wq4, int32_t M, int32_t N, int32_t K,
                               int32_t group, int32_t *acc, w4a4_stream stream);

/* Low-bit KV cache (Atom summary page, Summary paragraph 2: the KV cache is
 * kept in low bit-width; the NQKV abstract on the "smoothquant" tag page
 * quantizes it block by block). Each (token, head) vector of D channels is
 * one block of the layer's symmetric quantizer: s = fp32(absmax / qmax),
 * q = round-half-even of the correctly rounded x / s, qmax 7 (bits 4) or 127
 * (bits 8).
 *   X       device fp16 [T, ldx]: token t's head h is X[t, h D .. h D + D)
 *           (ldx >= H D, ldx % 8 == 0, 16-byte aligned)
 *   slot_mapping device int32 [T]: the cache slot of each token, or NULL for
 *           slot = t (then num_slots >= T). A slot outside [0, num_slots) is
 *           skipped (nothing written).
 *   cache_q device bytes [num_slots, H, D * bits / 8] (16-byte aligned): INT4
 *           codes two per byte, low nibble first, or INT8 codes
 *   cache_s device fp32 [num_slots, H]
 * D in {64, 128, 256} (else UNSUPPORTED); bits in {4, 8}. */
w4a4_status w4a4_kv_quant(const void *X, int64_t ldx, int32_t T, int32_t H, int32_t D, int32_t bits,
                          const int32_t *slot_mapping, int64_t num_slots, void *cache_q, float *cache_s,
                          w4a4_stream stream);

/* Gather of T tokens from the cache back to fp16: Y[t, h D + c] =
 * fp16(fp32(s * q)) (one correctly rounded fp32 product, then round to
 * nearest even) for the slot slot_mapping[t] (NULL: slot t); a slot outside
 * [0, num_slots) reads as zeros. Y device fp16 [T, ldy], ldy >= H D,
 * 16-byte aligned with ldy % 8 == 0. Same cache arguments and constraints as
 * w4a4_kv_quant. */
w4a4_status w4a4_kv_dequant(const void *cache_q, const float *cache_s, int64_t num_slots,
                            const int32_t *slot_mapping, int32_t T, int32_t H, int32_t D, int32_t bits,
                            void *Y, int64_t ldy, w4a4_stream stream);

/* Bytes of device workspace w4a4_select_outliers needs (0 for arguments it
 * would reject). A pure function of rows and K. */
size_t w4a4_select_outliers_workspace_bytes(int32_t rows, int32_t K);

/* Offline outlier-channel selection, the step before w4a4_make_perm (the
 * Atom summary page keeps a small set of outlier channels in 8 bits after
 * reordering them to a contiguous tail, Summary paragraph 2 and Interesting
 * ideas I1; neither page gives the rule that chooses them). Score of channel
 * c = max over the rows r of |Xcal[r, c]| (exact); the n_out channels with
 * the highest scores are selected, a tie going to the lower channel index.
 *   Xcal        device fp16 [rows, ldx], a calibration batch; rows may be 0
 *               (every score 0: channels 0 .. n_out-1)
 *   outlier_idx device int32 [n_out]: the selected channels, ascending
 *               (NULL allowed when n_out == 0)
 *   perm        device int32 [K]: the unselected channels ascending, then the
 *               selected ones ascending (what w4a4_make_perm returns for
 *               outlier_idx)
 *   chan_absmax device fp16 [K] (may be NULL): the scores
 *   workspace   device, >= w4a4_select_outliers_workspace_bytes(rows, K),
 *               256-byte aligned; no contents are required on entry
 * Xcal must be finite. INVALID_ARG for n_out outside [0, K], ldx < K, or a
 * NULL required pointer; ALIGNMENT unless Xcal is 16-byte aligned with
 * ldx % 8 == 0; UNSUPPORTED for K > 32768; WORKSPACE for a short workspace.
 * Three launches on `stream`. */
w4a4_status w4a4_select_outliers(const void *Xcal, int64_t ldx, int32_t rows, int32_t K,
                                 int32_t n_out, int32_t *outlier_idx, int32_t *perm,
                                 void *chan_absmax, void *workspace, size_t workspace_bytes,
                                 w4a4_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A4_H */
