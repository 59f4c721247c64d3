/*
 * vdtq.h -- C ABI of the MI355X (gfx950) hot path of 6Bit-Diffusion's
 * inference-time mixed-precision quantization for video diffusion
 * transformers (DMPQ + temporal delta cache + purified delta refresh).
 *
 * Pages cited by title and section:
 *   [gist] gist.science, "6Bit-Diffusion: Inference-Time Mixed-Precision
 *          Quantization for Video Diffusion Models", §2.A DMPQ, §2.B TDC,
 *          §2.C PDR, §4 results.
 *   [yly]  youleyou.com, "清华大学6Bit-Diffusion技术实现视频生成AI模型3倍压缩与速度翻倍",
 *          §一 DMPQ, §二 TDC, §三 PDR, §四 engineering, §七 limitations.
 *
 * Conventions shared by every call:
 *   - Every function returns VDTQ_OK (0) or an error code.  Arguments are
 *     validated before anything is enqueued: a non-zero return means no work
 *     was launched and no output was touched.  vdtq_last_error() returns a
 *     thread-local message for the last failing call on this thread.
 *   - Pointers named *_dev are device pointers (HBM of the current HIP
 *     device); all others are host pointers.  The caller allocates and frees
 *     every buffer; the library allocates nothing.
 *   - GPU work is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  Device faults surface at the caller's next synchronisation.
 *   - Device pointers must be 16-byte aligned.  Matrices are row-major.
 *   - Inputs must be finite; non-finite inputs give unspecified (but memory
 *     safe) outputs.
 *   - Calls on the same stream that share a workspace run in stream order;
 *     concurrent calls on different streams need distinct workspaces.
 *
 * Element formats:
 *   bf16    activations/weights/deltas, raw uint16 bit patterns.
 *   NVFP4   codes: 4-bit E2M1 (OCP MX FP4; 1 sign, 2 exponent, 1 mantissa,
 *           magnitudes 0,.5,1,1.5,2,3,4,6), two per byte, element 2j in the
 *           low nibble of byte j, rows of K/2 bytes.  Scales: one OCP E4M3
 *           ("fn": bias 7, max 448, no inf) byte per 16 consecutive elements
 *           of a row, rows of K/16 bytes.  Tensor scale: fp32 pair
 *           {amax_T, gs}; value = e2m1(code) * e4m3(scale) * gs.
 *   INT8    codes int8 [M][K] in [-127, 127], per-row fp32 scale s_m;
 *           value = q * s_m.
 *   MXFP4   OCP Microscaling v1.0: E2M1 codes packed as for NVFP4, one E8M0
 *           byte per 32 consecutive elements of a row (rows of K/32 bytes);
 *           value = e2m1(code) * 2^(byte - 127).  No tensor scale.
 *   MXFP8   the same with one E4M3 byte per element (rows of K bytes);
 *           value = e4m3(code) * 2^(byte - 127).
 */
#ifndef VDTQ_H
#define VDTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status codes */
#define VDTQ_OK 0
#define VDTQ_EINVAL 1        /* null pointer, bad shape/alignment/flag       */
#define VDTQ_EUNSUPPORTED 2  /* valid but outside what this build handles    */
#define VDTQ_EHIP 3          /* a HIP runtime call or launch failed          */

/* ------------------------------------------------------------ enums */
#define VDTQ_FMT_NVFP4 0
#define VDTQ_FMT_INT8 1
#define VDTQ_FMT_BF16 2      /* rotated activations in bf16 (W4A16 fallback) */
#define VDTQ_FMT_MXFP4 3     /* MX-native variant of NVFP4                   */
#define VDTQ_FMT_MXFP8 4     /* MX-native variant of INT8 (E4M3 elements)    */

#define VDTQ_OUT_BF16 0
#define VDTQ_OUT_F32 1

/* hadamard_quantize flags */
#define VDTQ_AMAX_GIVEN 1u   /* tensor_scale_dev[0] holds amax_T on entry    */
#define VDTQ_STATS 2u        /* write the four outlier statistics            */
#define VDTQ_GELU 4u         /* map X through GELU (bf16 result) first       */

/* scheduler actions */
#define VDTQ_ACT_SKIP 0
#define VDTQ_ACT_NVFP4 1
#define VDTQ_ACT_INT8 2
#define VDTQ_ACT_BF16 3

/* vdtq_workspace_bytes op ids */
#define VDTQ_OP_HADAMARD_QUANTIZE 0
#define VDTQ_OP_BLOCK_STATS 1
#define VDTQ_OP_QGEMM 2          /* vdtq_workspace_bytes(VDTQ_OP_QGEMM, M, N) */

const char* vdtq_last_error(void);
const char* vdtq_version(void);

/* Bytes of workspace a call needs for the given problem size (0 if none).
 * The (M, K) arguments are (rows, row length) for hadamard_quantize,
 * (n, ignored) for block_stats and (M, N) for the two GEMMs. */
size_t vdtq_workspace_bytes(int op, int64_t M, int64_t K);

/*
 * hadamard_quantize -- online block Hadamard transform of bf16 activations
 * followed by NVFP4 or per-token INT8 quantization (or, for the
 * full-precision fallback, bf16 rounding), with the outlier statistics fused
 * in.
 *
 * Defined by: [gist] §2.A (block Hadamard before quantization; NVFP4 for
 * stable blocks, INT8 for volatile ones), [yly] §一 (same), [yly] §三 (the
 * max/mean outlier ratio of the input), [yly] §四 / [gist] §4 (quantization
 * fused with the Hadamard transform in one kernel).
 *
 * Computes, per row of X and per block of `had_block` consecutive elements,
 * y = x * H_b / sqrt(b) (Sylvester H_b, butterflies h = 1, 2, ..., b/2 in
 * fp32 round-to-nearest-even), then:
 *   NVFP4: amax_T = max|Y| (computed, or read from tensor_scale_dev[0] when
 *     flags has VDTQ_AMAX_GIVEN); amax_T non-finite or < 2^-100 => all codes
 *     and scales 0, gs = 1.  Else gs = RN(amax_T / 2688), d = RN(6 gs); per
 *     16-group s8 = E4M3(RN(max|y| / d)) (nearest-even, saturating),
 *     s_dec = RN(e4m3(s8) * gs); code = E2M1(RN(y * RN(1 / s_dec)))
 *     (nearest-even, saturating, sign copied), 0 if s_dec == 0.
 *   INT8: per row a = max|y|; a non-finite or < 2^-100 => scale 0, codes 0;
 *     else s = RN(a / 127), q = rint_even(RN(y * RN(1 / s))), |q| <= 127.
 *   BF16: q = bf16_RNE(y) ([gist] §2.C: a flagged step runs in FP16/BF16;
 *     the weights exist only rotated, so the activations are rotated too).
 *   MXFP4 / MXFP8 (the MX-native variant of the two activation formats, for
 *     block-scaled matrix instructions; OCP Microscaling v1.0 §6.3): per
 *     32-element block, e = floor(log2 max|y|) - emax (emax 2 for E2M1, 8 for
 *     E4M3) clamped to [-127, 127] (-127 for an all-zero block), scale byte
 *     e + 127, element = nearest-even encoding of y / 2^e, saturating at 6
 *     or 448, sign copied.
 *
 * x_dev          bf16 [M][ldx], ldx >= K (elements); finite values whose
 *                transform stays finite (a NaN or an infinity, in X or
 *                from butterflies that overflow fp32, gives unspecified
 *                codes, scales and statistics; every access still stays
 *                inside the buffers)
 * M              rows (tokens), >= 0; M == 0 is a no-op (NVFP4 still writes
 *                the tensor scale {0, 1} unless AMAX_GIVEN)
 * K              columns, > 0, multiple of 16 and of had_block; for INT8,
 *                K <= 16384; for MXFP4 / MXFP8 a multiple of 32
 * had_block      16, 32, 64, 128 or 256
 * fmt            VDTQ_FMT_NVFP4, VDTQ_FMT_INT8, VDTQ_FMT_BF16, VDTQ_FMT_MXFP4
 *                or VDTQ_FMT_MXFP8
 * flags          VDTQ_AMAX_GIVEN (NVFP4 only) | VDTQ_STATS | VDTQ_GELU.
 *                VDTQ_GELU: every element is first replaced by
 *                bf16_RNE(GELU(x)), GELU in its tanh form evaluated in fp32
 *                by fixed steps: u = C0 (x + C1 x^3) (as (x*x)*x),
 *                z = clamp(-2u, -80, 90), GELU = x / (1 + exp(z)) with a
 *                correctly rounded division, C0 = RN(sqrt(2/pi)),
 *                C1 = RN(0.044715); exp(z) = 2^k p(r), k = rint(z RN(1/ln 2)),
 *                r = (z - k ln2_hi) - k ln2_lo (ln2_hi = 0x1.62ep-1,
 *                ln2_lo = 0x1.0bfbe8p-15), p the degree-7 Taylor polynomial
 *                with coefficients RN(1/n!) in Horner form, 2^k applied as
 *                2^floor(k/2) then 2^(k - floor(k/2)).  This is the DiT
 *                feed-forward's activation: quantizing FFN-up's bf16 output
 *                for FFN-down ([gist] §4: quantization fused with the
 *                kernels around it).  The statistics then describe GELU(x).
 *                The bf16 results come from a 7.3 KB lookup table in the
 *                library's device memory, one per GPU: the first call with
 *                VDTQ_GELU on a GPU builds it on `stream` and waits for it
 *                (once per GPU and process); later calls only read it.  A
 *                call on a capturing stream records the build into the
 *                graph instead of waiting.
 * q_dev          NVFP4, MXFP4: uint8 [M][K/2]; INT8: int8 [M][K]; BF16:
 *                bf16 [M][K]; MXFP8: uint8 E4M3 [M][K]
 * scales_dev     NVFP4: uint8 E4M3 [M][K/16]; INT8: float [M]; MXFP4,
 *                MXFP8: uint8 E8M0 [M][K/32]; BF16: ignored, may be NULL
 * tensor_scale_dev  NVFP4: float[2] {amax_T, gs} (amax_T is read when
 *                AMAX_GIVEN, else written); other formats: ignored, may be
 *                NULL
 * stats_dev      double[4] {max|x|, sum|x|, max|y|, sum|y|} when
 *                VDTQ_STATS (x before, y after the transform), else ignored
 * ws_dev/ws_bytes  workspace of vdtq_workspace_bytes(VDTQ_OP_HADAMARD_QUANTIZE,
 *                M, K) bytes (needed for NVFP4 without AMAX_GIVEN and with
 *                VDTQ_STATS; otherwise ignored, may be NULL)
 * Errors: VDTQ_EINVAL for null pointers, misalignment, bad sizes/flags or a
 * short workspace; VDTQ_EUNSUPPORTED for INT8 with K > 16384.
 */
int hadamard_quantize(const void* x_dev, int64_t M, int64_t K, int64_t ldx,
                      int had_block, int fmt, unsigned flags, void* q_dev,
                      void* scales_dev, float* tensor_scale_dev,
                      double* stats_dev, void* ws_dev, size_t ws_bytes,
                      void* stream);

/*
 * hadamard_quantize_noalloc -- hadamard_quantize without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same operation, arguments, outputs and errors as hadamard_quantize, minus
 * ws_dev/ws_bytes.  The per-workgroup partials live in a
 * library-owned device array of VDTQ_NOALLOC_SCRATCH_BYTES, one per GPU,
 * held from the first call on that GPU until the process ends; the call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * Everything in that array is written before it is read within a call, so
 * no state carries over between calls; but every call on one GPU shares the
 * array, so calls that overlap in time on one GPU (different streams, or
 * host threads racing on one device) race on it and give undefined
 * results.  Calls on one stream run in order and are safe.
 * Errors: those of hadamard_quantize; VDTQ_EUNSUPPORTED when the call would
 * need more than VDTQ_NOALLOC_SCRATCH_BYTES
 * (vdtq_workspace_bytes(VDTQ_OP_HADAMARD_QUANTIZE, M, K) above it: about
 * 36 bytes per 8192 elements or per row, whichever is more, i.e. up to
 * about 1.9e9 elements or 233k rows); VDTQ_EHIP if the array's device
 * address cannot be obtained.
 */
#define VDTQ_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int hadamard_quantize_noalloc(const void* x_dev, int64_t M, int64_t K, int64_t ldx,
                              int had_block, int fmt, unsigned flags, void* q_dev,
                              void* scales_dev, float* tensor_scale_dev,
                              double* stats_dev, void* stream);

/*
 * qgemm_w4a4 -- Y = gs_a * gs_w * (A_hat W_hat^T) + bias with NVFP4
 * activations A [M][K] and NVFP4 weights W [N][K] (both rotated by the same
 * block Hadamard transform along K, so Y is the linear layer's output).
 *
 * Defined by: [gist] §2.A and §3.1 (NVFP4 activations for stable blocks),
 * [gist] §4 / [yly] §四 (4-bit weights throughout: W4A4 ... W4A8).
 *
 * A_hat = e2m1(code) * e4m3(scale) per element (exact), W_hat likewise;
 * products and sums in fp32 (any order), result rounded to out_dtype.
 * Scale bytes are non-negative E4M3 values (0x00 .. 0x7E), as
 * hadamard_quantize writes them; a byte with the sign bit set gives
 * unspecified (memory-safe) results.
 *
 * a_q_dev  uint8 [M][K/2]   a_s_dev uint8 [M][K/16]   a_ts_dev float[2] {amax, gs}
 * w_q_dev  uint8 [N][K/2]   w_s_dev uint8 [N][K/16]   w_ts_dev float[2] {amax, gs}
 * bias_dev float [N] or NULL
 * y_dev    out_dtype [M][ldy], ldy >= N (elements)
 * M, N >= 0 (0 is a no-op); K > 0, multiple of 16.
 * ws_dev/ws_bytes  workspace of vdtq_workspace_bytes(VDTQ_OP_QGEMM, M, N)
 *   bytes, 256-byte aligned: fp32 partial sums of output tiles split along
 *   K (the tiles of a partial last wave), added in a fixed order.  No
 *   initial contents are needed; calls on one stream may share it,
 *   concurrent calls need distinct workspaces.
 */
int qgemm_w4a4(const uint8_t* a_q_dev, const uint8_t* a_s_dev,
               const float* a_ts_dev, const uint8_t* w_q_dev,
               const uint8_t* w_s_dev, const float* w_ts_dev,
               const float* bias_dev, void* y_dev, int64_t ldy, int out_dtype,
               int64_t M, int64_t N, int64_t K, void* ws_dev, size_t ws_bytes,
               void* stream);

/*
 * qgemm_w4a8 -- Y[m][n] = s_a[m] * gs_w * sum_k q_a[m][k] W_hat[n][k] + bias
 * with per-token INT8 activations and NVFP4 weights.
 *
 * Defined by: [gist] §2.A (INT8 for volatile blocks), [yly] §三 (INT8 for
 * the first recompute after a skip), [gist] §4 (W4A8 operating point).
 *
 * Every product q * W_hat is exact and accumulated in fp32; with all weight
 * scales 1 (E4M3 byte 0x38), gs_w = 1 and s_a = 1 the result equals the
 * integer sum_k q_a * e2m1(w) exactly while partial sums stay below 2^24.
 *
 * a_q_dev int8 [M][K]   a_s_dev float [M]   weights, workspace as in
 * qgemm_w4a4.
 */
int qgemm_w4a8(const int8_t* a_q_dev, const float* a_s_dev,
               const uint8_t* w_q_dev, const uint8_t* w_s_dev,
               const float* w_ts_dev, const float* bias_dev, void* y_dev,
               int64_t ldy, int out_dtype, int64_t M, int64_t N, int64_t K,
               void* ws_dev, size_t ws_bytes, void* stream);

/*
 * qgemm_w4a16 -- Y = gs_w * (A W_hat^T) + bias with bf16 activations: the
 * full-precision fallback of a step whose input fails the outlier check.
 *
 * Defined by: [gist] §2.C and [yly] §三 (full precision, FP16/BF16, for a
 * step flagged by the max/mean outlier ratio before its delta is cached),
 * [gist] §4 (the weights stay 4-bit: the memory figure).
 *
 * A = the rotated activations in bf16 (hadamard_quantize with
 * VDTQ_FMT_BF16); W_hat = e2m1(code) * e4m3(scale), exact in bf16; products
 * exact, accumulated in fp32 (any order), result rounded to out_dtype.
 *
 * a_dev    bf16 [M][K], 16-byte aligned
 * w_q_dev, w_s_dev, w_ts_dev   NVFP4 weights as in qgemm_w4a4 (w_s_dev
 *          4-byte aligned)
 * bias_dev float [N] or NULL; y_dev out_dtype [M][ldy], ldy >= N
 * M, N >= 0 (0 is a no-op); K > 0, multiple of 16.
 * ws_dev/ws_bytes  workspace of vdtq_workspace_bytes(VDTQ_OP_QGEMM, M, N)
 *          bytes, 256-byte aligned, as for qgemm_w4a4 (partial sums of the
 *          tiles of a partial last wave, split along K).
 * Errors: VDTQ_EINVAL as for the other GEMMs (a short workspace included);
 * VDTQ_EUNSUPPORTED when K is not a multiple of 64 or an operand reaches
 * 4 GB.
 */
int qgemm_w4a16(const void* a_dev, const uint8_t* w_q_dev,
                const uint8_t* w_s_dev, const float* w_ts_dev,
                const float* bias_dev, void* y_dev, int64_t ldy,
                int out_dtype, int64_t M, int64_t N, int64_t K,
                void* ws_dev, size_t ws_bytes, void* stream);

/*
 * qgemm_mx -- the MX-native variant of qgemm_w4a4 / qgemm_w4a8:
 * Y = A_hat W_hat^T + bias with MXFP4 weights and MXFP4 (4-bit) or MXFP8
 * (E4M3, 8-bit) activations, both produced by hadamard_quantize with the
 * same had_block, run on CDNA4's block-scaled matrix instruction.
 *
 * Defined by: [gist] §2.A / §3.1 and §4 (4-bit weights; 4- or 8-bit
 * activations per block and step) with the operands in the OCP
 * Microscaling v1.0 formats ([gist] §2.A names NVFP4 as a Blackwell format;
 * this variant is the one CDNA4's matrix cores read without decoding).
 * A_hat = element * 2^(scale byte - 127) per 32-element block, W_hat
 * likewise; products of the elements are exact, sums are in fp32 inside
 * the matrix instruction (E4M3 x E2M1 sums are not rounded per add: the
 * instruction's own accumulation order and alignment apply).
 *
 * a_fmt          VDTQ_FMT_MXFP4 or VDTQ_FMT_MXFP8
 * a_q_dev        MXFP4: uint8 [M][K/2]; MXFP8: uint8 E4M3 [M][K]
 * a_s_dev        uint8 E8M0 [M][K/32] (4-byte aligned)
 * w_q_dev        uint8 [N][K/2] E2M1 codes; w_s_dev uint8 E8M0 [N][K/32]
 * bias_dev       float [N] or NULL
 * y_dev/ldy/out_dtype  as for qgemm_w4a4
 * ws_dev/ws_bytes  workspace of vdtq_workspace_bytes(VDTQ_OP_QGEMM, M, N)
 *                bytes, 256-byte aligned (partial sums of split tiles)
 * Errors: VDTQ_EINVAL for a bad a_fmt, K not a multiple of 32, null or
 * misaligned pointers, ldy < N or a short workspace; VDTQ_EUNSUPPORTED for
 * K not a multiple of 128 or an operand matrix of 4 GB or more.
 */
int qgemm_mx(int a_fmt, const uint8_t* a_q_dev, const uint8_t* a_s_dev,
             const uint8_t* w_q_dev, const uint8_t* w_s_dev,
             const float* bias_dev, void* y_dev, int64_t ldy, int out_dtype,
             int64_t M, int64_t N, int64_t K, void* ws_dev, size_t ws_bytes,
             void* stream);

/*
 * qgemm_mx_quant -- qgemm_mx whose output never reaches HBM in bf16: the
 * epilogue turns each finished tile into the next linear's MX activation.
 * For FFN-up it computes, per output row, exactly what
 *   Y = qgemm_mx(A, W, bias) in bf16, then
 *   hadamard_quantize(Y, 64, out_fmt, flags) (VDTQ_GELU: GELU first)
 * would produce for FFN-down, in one kernel.
 *
 * Defined by: [gist] §4 and [yly] §四 (quantization fused with the kernels
 * around it, so that low-precision activations do not make an extra round
 * trip through memory), over the operations of qgemm_mx and
 * hadamard_quantize; GELU is the DiT feed-forward's activation between
 * FFN-up and FFN-down.
 *
 * Per row m and per 64-column chunk of Y: y = bf16_RNE(acc + bias) with acc
 * the fp32 sum of qgemm_mx (bit-identical to qgemm_mx's bf16 output when
 * that call does not split tiles along K), optional GELU as in
 * hadamard_quantize, the 64-point Hadamard transform, MX encoding.
 *
 * a_fmt          VDTQ_FMT_MXFP4 or VDTQ_FMT_MXFP8 (the GEMM's activations)
 * a_q_dev .. bias_dev  as for qgemm_mx; bias 16-byte aligned
 * had_block      64 (the transform of the output rows)
 * out_fmt        VDTQ_FMT_MXFP4 or VDTQ_FMT_MXFP8 (the next activation)
 * flags          0 or VDTQ_GELU
 * q_out_dev      MXFP4: uint8 [M][N/2]; MXFP8: uint8 E4M3 [M][N]
 *                (16-byte aligned)
 * s_out_dev      uint8 E8M0 [M][N/32] (4-byte aligned)
 * M, N, K        as for qgemm_mx; N a multiple of 64
 * No workspace: tiles are never split along K on this path.  VDTQ_GELU
 * uses the GPU's GELU table as hadamard_quantize does (built and waited for
 * by the first call that needs it on the GPU).
 * Errors: VDTQ_EINVAL for bad formats or flags, N not a multiple of 64, K
 * not a multiple of 32, null or misaligned pointers; VDTQ_EUNSUPPORTED for
 * had_block other than 64, K not a multiple of 128 or an operand matrix of
 * 4 GB or more.
 */
int qgemm_mx_quant(int a_fmt, const uint8_t* a_q_dev, const uint8_t* a_s_dev,
                   const uint8_t* w_q_dev, const uint8_t* w_s_dev,
                   const float* bias_dev, int had_block, int out_fmt,
                   unsigned flags, uint8_t* q_out_dev, uint8_t* s_out_dev,
                   int64_t M, int64_t N, int64_t K, void* stream);

/*
 * block_stats -- one pass over a block's input, output and cached delta.
 *
 * Defined by: [gist] §2.A (Gamma_{t-1}: relative input-output difference of
 * the block), [gist] §2.B (similarity of Delta_{t-1} and Delta_{t-2}; the
 * cached residual delta), [yly] §三 (max/mean outlier ratio), [yly] §七
 * (the online metrics cost a pass; keep it cheap).
 *
 * d = RN_fp32(out - in); dnew = bf16_RNE(d) (written when dnew_dev != NULL).
 * stats_dev double[8] = {sum d^2, sum in^2, sum (dnew - dprev)^2,
 *   sum dprev^2, max|in|, sum|in|, max|out|, sum|out|}; entries 2 and 3 are
 *   0 when dprev_dev == NULL.  Sums are accumulated in fp64 in a fixed
 *   order (bit-identical across runs).
 * in_dev, out_dev, dprev_dev, dnew_dev: bf16 [n] (dnew may not alias dprev)
 * n >= 0 (n == 0 writes zeros).
 * ws_dev: vdtq_workspace_bytes(VDTQ_OP_BLOCK_STATS, n, 1) bytes, 16-byte
 *   aligned.  Its first 4 bytes are a completion counter (the last
 *   workgroup to finish reduces the per-workgroup partials, in a fixed
 *   order): they must be zero before the first call that uses the
 *   workspace, and every completed call leaves them zero.  Use this
 *   workspace for block_stats / block_stats_mx8 calls only (other entry
 *   points write theirs from the start); calls sharing it run in stream
 *   order.
 */
int block_stats(const void* in_dev, const void* out_dev,
                const void* dprev_dev, void* dnew_dev, int64_t n,
                double* stats_dev, void* ws_dev, size_t ws_bytes,
                void* stream);

/*
 * block_stats_mx8 -- block_stats with the delta cache in MXFP8.
 *
 * Defined by: the passages of block_stats, and [yly] §七 (the temporal
 * delta cache needs extra memory, which storing it in low precision
 * reduces).
 *
 * d = RN_fp32(out - in); Delta_new = MXFP8(d): per 32 consecutive elements
 * e = floor(log2 max|d|) - 8 clamped to [-127, 127] (-127 for an all-zero
 * block), code = E4M3 nearest-even of d / 2^e saturating at 448 (sign kept),
 * scale byte e + 127 (the MX conversion of hadamard_quantize's MXFP8).
 * stats_dev double[8] as for block_stats, except that entries 2 and 3 are
 * taken on the dequantized stored deltas: sum (dnew - dprev)^2 and
 * sum dprev^2 with dnew, dprev = e4m3(code) * 2^(byte - 127).
 * in_dev, out_dev  bf16 [n], n a multiple of 32 (16-byte aligned)
 * dprev_q_dev, dprev_s_dev  the previous delta: uint8 E4M3 [n] (8-byte
 *                aligned) and uint8 E8M0 [n/32], both NULL when there is none
 * dnew_q_dev, dnew_s_dev  the new delta, same layout; both NULL to skip the
 *                write; must not alias dprev
 * ws_dev: as for block_stats (zeroed completion counter first).
 * Errors: VDTQ_EINVAL for n not a multiple of 32, a null or misaligned
 * pointer, codes without scales (or the reverse), aliasing, or a short
 * workspace.
 */
int block_stats_mx8(const void* in_dev, const void* out_dev,
                    const uint8_t* dprev_q_dev, const uint8_t* dprev_s_dev,
                    uint8_t* dnew_q_dev, uint8_t* dnew_s_dev, int64_t n,
                    double* stats_dev, void* ws_dev, size_t ws_bytes,
                    void* stream);

/* ------------------------------------------------------------ scheduler */

typedef struct {
  double gamma;    /* Gamma threshold: NVFP4 below, INT8 at or above        */
  double tau;      /* skip only when r < tau ...                            */
  double tau_acc;  /* ... and acc + r < tau_acc (error accumulator)         */
  double rho;      /* BF16 when the input outlier ratio exceeds rho         */
  double tau_u;    /* BF16 when r exceeds tau_u (+inf disables)             */
  int32_t warmup;  /* no skip before this step index                        */
  int32_t pad_;
} vdtq_dmpq_params;

typedef struct {
  int64_t step;
  int32_t has_d1, has_d2, skipped_last, has_gamma;
  double gamma_prev, r_last, acc;
} vdtq_dmpq_state;

/* Fresh state (step 0, no history, r_last = +inf). */
void dmpq_state_init(vdtq_dmpq_state* s);

/*
 * dmpq_step -- host-side per-block decision for one denoising step.
 *
 * Defined by: [gist] §2.A (low Gamma -> NVFP4, high -> INT8), [gist] §2.B
 * (skip on Delta similarity; error-guided switching refreshes the cache),
 * [gist] §2.C and [yly] §三 (outliers or temporal uncertainty -> full
 * precision before a cache write), [yly] §三 (restart after a skip -> INT8).
 *
 * last_stats: host double[8] from block_stats of the previous step if that
 *   step was computed, NULL otherwise.  in_ratio: outlier ratio
 *   max|x| / mean|x| of the block input at this step.
 * 1. If last_stats: Gamma_prev = sqrt(s0/s1) (0 if s0 = s1 = 0, +inf if only
 *    s1 = 0); if a delta was already cached, r_last = sqrt(s2/s3) (+inf if
 *    s3 = 0); the delta history shifts; skipped_last = 0; acc = 0.
 * 2. SKIP if step >= warmup, two deltas are cached, r_last < tau and
 *    acc + r_last < tau_acc; then acc += r_last, skipped_last = 1.
 * 3. Else BF16 if in_ratio > rho or (two deltas cached and r_last > tau_u);
 *    else INT8 if skipped_last or no Gamma yet or Gamma_prev >= gamma;
 *    else NVFP4.
 * Pure host code, deterministic; *action receives VDTQ_ACT_*.
 */
int dmpq_step(const vdtq_dmpq_params* p, vdtq_dmpq_state* s,
              const double* last_stats, double in_ratio, int* action);

/* max / (sum / n); 1 when sum == 0 or n == 0. */
double vdtq_outlier_ratio(double max_abs, double sum_abs, int64_t n);

/*
 * dmpq_budget_gamma -- the Gamma threshold of one denoising step in
 * bit-budget mode.
 *
 * Defined by: [gist] §2.A and [yly] §一 (Gamma_{t-1} of a block predicts the
 * precision its linears need: high -> INT8, low -> NVFP4) and [yly] §四 (the
 * W4A6 operating point averages 6 activation bits).
 *
 * Ranks the blocks by Gamma_{t-1}: with k = floor(n * (avg_bits - 4) / 4)
 * clamped to [0, n], returns the k-th largest of gammas[0..n-1] (+inf when
 * k = 0), to be passed as params.gamma to every dmpq_step of the step, so
 * that the k most sensitive blocks run INT8 and the others NVFP4.  Blocks
 * tied at the boundary all take INT8 (Gamma >= gamma).  The restart INT8,
 * BF16 and skips are decided by dmpq_step as usual, outside the budget.
 * gammas: host double[n], no NaN (+inf allowed).  Returns +inf when
 * gammas == NULL, n <= 0 or avg_bits is not finite.  Allocates nothing.
 */
double dmpq_budget_gamma(const double* gammas, int32_t n, double avg_bits);

/*
 * dmpq_depth_params -- one block's scheduler parameters under a depth-aware
 * caching profile.
 *
 * Defined by: [yly] §五 (blocks at different depths of the transformer have
 * different temporal stability, the basis the page gives for a layered,
 * adaptive caching policy) over the skip rule of dmpq_step ([gist] §2.B).
 *
 * *out = *base except that, with d = depth / (n_blocks - 1) (0 when
 * n_blocks == 1) and s = s_shallow + (s_deep - s_shallow) * d (double,
 * in that order), out->tau = base->tau * s and out->tau_acc =
 * base->tau_acc * s: the skip thresholds move linearly with relative
 * depth from s_shallow at the first block to s_deep at the last.  gamma,
 * rho, tau_u and warmup are copied unchanged.  s_shallow = s_deep = 1 gives
 * *base back.  out may alias base.
 * Errors: VDTQ_EINVAL for a null pointer, n_blocks <= 0, depth outside
 * [0, n_blocks), or a factor that is negative or not finite (out untouched).
 * Pure host code; allocates nothing.
 */
int dmpq_depth_params(const vdtq_dmpq_params* base, int32_t depth, int32_t n_blocks,
                      double s_shallow, double s_deep, vdtq_dmpq_params* out);

#ifdef __cplusplus
}
#endif
#endif /* VDTQ_H */
