/*
 * mxgemm.h - C ABI of the MI355X (gfx950) block-scaled matrix multiply library.
 *
 * The operation:  C[i][j] = sum_b 2^(sA[i][b]-127) * 2^(sB[j][b]-127)
 *                           * sum_{k in block b} a[i][k] * b[j][k]
 * with A (M x K) and B (N x K) stored as low-precision codes (FP8 E4M3, or FP4
 * E2M1 packed two per byte) plus one UE8M0 scale byte per 32 consecutive
 * K elements, and C (M x N) in fp32.  Operand model: "Metal tensors でカスタム
 * 機械学習オペレーションを最適化する" (WWDC26 session 330 summary), sections
 * "多平面 tensor" and "Scale Factor 付き量子化 tensor を作成する" - a data plane
 * plus an E8M0 scale plane with one scale per block of 32 along the innermost
 * (reduction) dimension; section "スライスと量子化行列乗算" - the quantized
 * matmul consumes both planes, dequantization included.  The same session's
 * transcript, "Metal 텐서로 맞춤형 머신 러닝 연산 최적화하기", chapters
 * "Multi-plane tensors" and "Quantized matrix multiplication".
 *
 * Conventions shared by every entry point:
 *   - All pointers are DEVICE pointers (hipMalloc / torch CUDA tensors) owned
 *     by the caller; the library never allocates, frees or retains them.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued asynchronously in stream order; nothing synchronizes.  A
 *     fault inside a kernel surfaces at the caller's next synchronization.
 *   - Arguments are validated before anything is launched; on error nothing is
 *     enqueued and a nonzero MXG_* status is returned.  No exceptions cross the
 *     ABI and nothing is printed.
 *   - Layouts are row-major.  Every operand row runs along K (K contiguous),
 *     so A is M x K and B is N x K ("transposed right operand"); the scale
 *     planes are M x K/32 and N x K/32 bytes, row-major, and use the same row
 *     order as their data planes.
 *   - E4M3 is the OCP "FN" variant (bias 7, max 448, NaN = S.1111.111, no
 *     infinity).  E5M2 is the OCP variant with IEEE-style specials (bias 15,
 *     max 57344, S.11111.00 = +-inf, S.11111.xx (xx != 0) = NaN).  E2M1 codes
 *     are packed with the even K index in the low nibble.  UE8M0 byte e means
 *     2^(e-127); e = 255 is NaN and propagates.
 *   - Data pointers (codes, fp16, fp32) must be 16-byte aligned (the kernels
 *     move operands with 16-byte loads); scale pointers need no alignment.
 *     The 128-byte row alignment the RIGEL summary reports for Metal inline
 *     tensors ("Resumo Técnico: RIGEL", section 3) is not required here.
 *   - The library runs on gfx950 only; other devices get MXG_EUNSUPPORTED.
 */
#ifndef MXGEMM_H
#define MXGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MXG_OK 0
#define MXG_EINVAL 1         /* null pointer, non-positive or oversized dim, K % 32 != 0, bad enum */
#define MXG_EALIGN 2         /* a data pointer is not 16-byte aligned */
#define MXG_EUNSUPPORTED 3   /* current device is not gfx950 */
#define MXG_EHIP 4           /* the HIP runtime reported an error at launch */

/* Element formats (float formats: values equal the MFMA operand-format
 * ids).  INT4 / INT2 are two's complement integer codes (-8..7 / -2..1): the
 * 4-bit and 2-bit integer tensor types of the WWDC26 session 330 summary,
 * section "量子化データ型のネイティブサポート", with the block-wise scale of its
 * section "2-bit 量子化の限界圧縮を探る".  INT4 codes are packed two per byte
 * (even K index in the low nibble), INT2 codes four per byte (K index k in
 * bits 2 (k mod 4)).  E2M3 / E3M2 are the FP6 operands of the scaled matrix
 * unit, taken with the OCP Microscaling definitions (the pages name the type
 * but no layout): E2M3 sign, 2 exponent bits (bias 1), 3 mantissa bits,
 * largest 7.5; E3M2 sign, 3 exponent bits (bias 3), 2 mantissa bits, largest
 * 28; no NaN or infinity codes; packed little-endian, element k at bits
 * 6k .. 6k+5 of its row (3 bytes per 4 elements). */
#define MXG_ELEM_E4M3 0
#define MXG_ELEM_E5M2 1
#define MXG_ELEM_E2M3 2
#define MXG_ELEM_E3M2 3
#define MXG_ELEM_E2M1 4
#define MXG_ELEM_INT4 8
#define MXG_ELEM_INT2 9

/* Operand-format pairs for mxgemm_run: (A element, B element). */
#define MXG_FMT_FP8_FP8 0   /* E4M3 x E4M3 */
#define MXG_FMT_FP8_FP4 1   /* E4M3 x E2M1 */
#define MXG_FMT_FP4_FP4 2   /* E2M1 x E2M1 */
#define MXG_FMT_BF8_BF8 3   /* E5M2 x E5M2 */
#define MXG_FMT_FP8_BF8 4   /* E4M3 x E5M2 */
#define MXG_FMT_BF8_FP8 5   /* E5M2 x E4M3 */
#define MXG_FMT_FP8_INT4 6  /* E4M3 activations x INT4 weights */
#define MXG_FMT_FP8_INT2 7  /* E4M3 activations x INT2 weights */
#define MXG_FMT_FP8_FP6 8   /* E4M3 activations x E2M3 (FP6) weights */
#define MXG_FMT_FP8_BF6 9   /* E4M3 activations x E3M2 (FP6) weights */

/* Largest accepted M, N (rows) and K. */
#define MXG_MAX_DIM (1 << 20)

/* Output element types and activations of mxgemm_run_fused / mxgemm_epilogue. */
#define MXG_OUT_F32 0    /* fp32 */
#define MXG_OUT_BF16 1   /* bfloat16 bits, uint16 per element */
#define MXG_OUT_F16 2    /* IEEE binary16 bits, uint16 per element */
#define MXG_ACT_NONE 0
#define MXG_ACT_GELU 1   /* GELU(y) = y * Phi(y), Phi the standard normal CDF */

/*
 * mxgemm_quantize - fp32 rows -> block-scaled codes plus UE8M0 scales.
 *
 * For every row r and every block b of 32 consecutive elements along K:
 *   amax = max |X[r][32b .. 32b+31]|;
 *   e    = floor(log2(amax)) - emax  (emax = 8 for E4M3, 15 for E5M2, 2 for
 *          E2M1, E2M3 and INT4, 4 for E3M2, 0 for INT2: the exponent of the
 *          largest power of two in the element range),
 *          clamped to [-127, 127]; e = -127 when amax = 0;
 *   S[r][b] = e + 127;
 *   Q[r][k] = round-to-nearest-even(X[r][k] * 2^-e), saturated to +-448
 *             (E4M3), +-57344 (E5M2), +-6 (E2M1), +-7.5 (E2M3), +-28 (E3M2),
 *             -8..7 (INT4) or -2..1 (INT2); float codes keep the sign
 *             (-0 -> 0x80 / 0x20 / 0x8).
 * A block holding a NaN or an infinity gets S = 255 (NaN) and zero codes.
 * E4M3 saturating rather than overflowing follows "Resumo Técnico: RIGEL",
 * section 3 (saturation); one E8M0 scale per 32 elements follows the WWDC26
 * session 330 summary, section "Scale Factor 付き量子化 tensor を作成する".
 * The exponent rule is the OCP Microscaling convention.
 *
 *   X     device, rows x K fp32, row-major, 16-byte aligned (read only)
 *   rows  >= 1;  K >= 32, K % 32 == 0
 *   elem  MXG_ELEM_E4M3 or MXG_ELEM_E5M2 (Q: rows x K bytes), MXG_ELEM_E2M1 or
 *         MXG_ELEM_INT4 (Q: rows x K/2 bytes, even k in the low nibble),
 *         MXG_ELEM_INT2 (Q: rows x K/4 bytes), MXG_ELEM_E2M3 or
 *         MXG_ELEM_E3M2 (Q: rows x 3K/4 bytes); Q 16-byte aligned (written)
 *   S     device, rows x K/32 bytes (written)
 * Returns MXG_OK or an error status.  The output is bit-for-bit deterministic.
 */
int mxgemm_quantize(const float *X, int64_t rows, int64_t K, int elem,
                    void *Q, uint8_t *S, void *stream);

/*
 * mxgemm_run - C = (A * 2^sA)(B * 2^sB)^T in fp32 on the scaled MFMA path.
 *
 *   A, scaleA  device; A is M x K codes (E4M3 / E5M2: M*K bytes; E2M1: M*K/2
 *              bytes), scaleA is M x K/32 UE8M0 bytes
 *   (B: N x K codes of its element format: INT4 N*K/2 bytes, INT2 N*K/4,
 *    FP6 3N*K/4)
 *   B, scaleB  device; B is N x K codes, scaleB is N x K/32 bytes
 *   C          device, M x N fp32 row-major, 16-byte aligned; overwritten
 *   M, N       >= 1 (any value; edges are masked); K >= 32, K % 32 == 0
 *   fmt        one of the MXG_FMT_* pairs (A element, B element)
 * Each 32-element block product is formed by CDNA4's scaled fp8/fp4 MFMA,
 * which applies the E8M0 scales itself; partial sums accumulate in fp32.
 * Integer weights (MXG_FMT_FP8_INT4 / _INT2) are fed to that MFMA as the
 * E4M3 / E2M1 codes of the same values (exact: -8..7 and -2..1 are values of
 * those formats), remapped in registers; they take the decode kernel (INT2:
 * K a multiple of 4096) and the split-K kernel, and with M > 64 the 4-wave
 * tiled kernel.  FP6 weights (MXG_FMT_FP8_FP6 / _BF6) are MFMA operands as stored
 * (the instruction's E2M3 / E3M2 modes: a lane's 32 codes are its 24 bytes of
 * a row); they take the decode kernel and the split-K kernel, and with
 * M > 64 the 4-wave tiled kernel when K % 128 == 0, else the split-K kernel
 * once per 64 rows of A.
 * Decode shapes with E4M3 activations and E4M3, E2M1 or FP6 weights take
 * weight-streaming kernels: for M <= 64 and K a multiple of 1024 from 2048,
 * one that reads B once per launch (fp32 C: all rows per launch, K in chunks
 * of up to 16384 (E2M1 weights) or 12288 (E4M3 and FP6 weights), fewer as M
 * grows, each chunk adding into C, K up to 131072; 16-bit C through
 * mxgemm_run_fused: all of K per launch, K up to 16384 / 12288, one launch per
 * 64, 32 or 16 rows for K <= 4096, <= 8192, above); for other small M
 * (M <= 64) a split-K kernel, which with fp32 C and M <= 16 only adds the
 * last K mod 1024 elements to the decode kernel's sum over the rest.
 * Result accuracy: |C - exact| <= K * 2^-24 * sum_k |a_ik b_jk|
 * + 2^-7 * sum_t max_{k in step t} |a_ik b_jk| (steps of 128 K elements,
 * products taken with their scales).  The second term is the scaled MFMA's
 * own: it adds a step's products in one operation and drops bits far below
 * the largest of them (measured at most 2^-8.6 of it per instruction; none
 * for E2M1 x E2M1).  It matters for short K or block scales that vary; on
 * long-K, same-magnitude data the first term alone holds.
 * Returns MXG_OK or an error status.  The result is deterministic.
 */
int mxgemm_run(const void *A, const uint8_t *scaleA,
               const void *B, const uint8_t *scaleB,
               float *C, int64_t M, int64_t N, int64_t K, int fmt, void *stream);

/*
 * mxgemm_run_fused - mxgemm_run with the output step fused into the GEMM's
 * epilogue: for every element, in fp32 with round-to-nearest-even,
 *   y = acc[i][j] + bias[j]        (when bias != NULL)
 *   y = GELU(y)                    (when act == MXG_ACT_GELU)
 *   C[i][j] = y in the type out_type (RNE; overflow -> +-inf; NaN stays NaN)
 * where acc is exactly what mxgemm_run writes for the same operands.  C then
 * makes a single trip to memory, at 2 bytes per element for bf16 / fp16:
 * the fused GEMM + bias + GELU kernel of "Resumo Técnico: RIGEL", section
 * "4. Oportunidades de Otimização".  GELU is evaluated as y/2 * (1 + erf(y /
 * sqrt 2)) with erf from Abramowitz & Stegun formula 7.1.26 (absolute error
 * <= 1.5e-7); GELU(-inf) is NaN.
 *
 *   A, scaleA, B, scaleB, M, N, K, fmt  as for mxgemm_run
 *   C         device, M x N row-major elements of out_type, 16-byte aligned;
 *             overwritten
 *   bias      device, N fp32 values, 16-byte aligned (read only), or NULL
 *   act       MXG_ACT_NONE or MXG_ACT_GELU
 *   out_type  MXG_OUT_F32, MXG_OUT_BF16 or MXG_OUT_F16
 * With bias == NULL, act == MXG_ACT_NONE and out_type == MXG_OUT_F32 the
 * result is bit-identical to mxgemm_run.  The result equals, bit for bit,
 * mxgemm_run followed by mxgemm_epilogue with the same bias / act / out_type.
 * Returns MXG_OK or an error status (MXG_EINVAL for an unknown act or
 * out_type, MXG_EALIGN for a misaligned C or bias).  Deterministic.
 */
int mxgemm_run_fused(const void *A, const uint8_t *scaleA,
                     const void *B, const uint8_t *scaleB,
                     void *C, int64_t M, int64_t N, int64_t K, int fmt,
                     const float *bias, int act, int out_type, void *stream);

/*
 * mxgemm_epilogue - the same output step as a separate pass over an fp32
 * matrix: Y[i][j] = out_type(act(X[i][j] + bias[j])), with the arithmetic
 * of mxgemm_run_fused.  The decomposed path the fused kernel is compared
 * with; also usable on any fp32 GEMM result.
 *
 *   X         device, M x N fp32 row-major, 16-byte aligned (read only)
 *   M, N      >= 1
 *   bias, act, out_type  as for mxgemm_run_fused
 *   Y         device, M x N elements of out_type, 16-byte aligned; may not
 *             overlap X unless Y == X and out_type == MXG_OUT_F32
 * Returns MXG_OK or an error status.  Deterministic.
 */
int mxgemm_epilogue(const float *X, int64_t M, int64_t N, const float *bias,
                    int act, int out_type, void *Y, void *stream);

/*
 * fp16gemm_run - dense fp16 comparison GEMM, fp32 accumulate and output.
 *
 *   A  device, M x K binary16 (uint16 bits), row-major, 16-byte aligned
 *   B  device, binary16; K x N row-major when b_is_nk == 0,
 *      N x K row-major (same layout as the MX operands) when b_is_nk == 1
 *   C  device, M x N fp32 row-major, 16-byte aligned; overwritten
 *   M, N >= 1; K >= 8, K % 8 == 0
 * This is the half-precision rung of "Treinar LLM em Swift: multiplicação de
 * matrizes do Gflop/s ao Tflop/s", section "Passo 6" (FP16 instead of FP32),
 * and the fp16 baseline against which "Resumo Técnico: RIGEL", section
 * "Metodologia: O Harness RIGEL", judges low precision as accelerated
 * (>= 1.5x fp16 throughput) or emulated.
 */
int fp16gemm_run(const uint16_t *A, const uint16_t *B, float *C,
                 int64_t M, int64_t N, int64_t K, int b_is_nk, void *stream);

/*
 * mxgemm_run_dequant_fp16 - ablation of mxgemm_run (same arguments, fmt must
 * be MXG_FMT_FP8_FP8): each operand fragment is dequantized in registers to
 * fp16 (code * 2^(scale-127), rounded to nearest-even fp16) and multiplied
 * with the fp16 MFMA.  This is the register-resident custom-dequantization
 * route of the WWDC26 session 330 transcript, chapter "Quantized matrix
 * multiplication" (dequantize into a cooperative tensor instead of bouncing
 * through threadgroup memory).  Exact only while every code * 2^(scale-127)
 * is an fp16 value (E4M3 scale bytes within [112, 134]); outside that range
 * fp16 rounding, overflow or underflow adds error.  Kept for measurement.
 */
int mxgemm_run_dequant_fp16(const void *A, const uint8_t *scaleA,
                            const void *B, const uint8_t *scaleB,
                            float *C, int64_t M, int64_t N, int64_t K, int fmt,
                            void *stream);

/*
 * mxgemm_mfma_ceiling - measurement helper (not part of the product path):
 * the matrix-core rate the chip sustains on given operand bytes with no
 * memory traffic, the measured ceiling reported beside the published peak
 * ("Resumo Técnico: RIGEL", section "Metodologia: O Harness RIGEL": compute
 * ceilings are triangulated by measurement, not taken from the data sheet).
 *
 * Every wave of `workgroups` workgroups of 8 waves (two per SIMD, like the
 * large GEMM) loads 12 operand fragments (32 bytes per lane, from positions
 * spread over `ops`) and, for kind MXG_FMT_*, 3 scale registers (from
 * `scales`), then runs `iters` rounds of the GEMM's compute phase: 32
 * 16x16x128 scaled MFMAs of that format pair (8 A x 4 B fragments).  For kind
 * MXG_CEIL_FP16 it runs 64 fp16 16x16x32 MFMAs per round on fp16 bits from
 * `ops` (scales unused).  Flops per launch: workgroups * 8 * iters * 32 *
 * 65536 (fp16: workgroups * 8 * iters * 64 * 16384).
 *
 *   ops          device, >= 32 bytes, 16-byte aligned (read only): operand codes
 *   scales       device, >= 4 bytes, 4-byte aligned (read only); NULL for fp16
 *   kind         MXG_FMT_* or MXG_CEIL_FP16
 *   iters        1 .. 2^30;  workgroups  1 .. 2^20
 *   out          device, workgroups * 512 floats, 16-byte aligned (written):
 *                per-lane sums of the accumulators (keeps the work live)
 *   clocks       device, workgroups * 2 uint32, 4-byte aligned (written), or
 *                NULL: for each workgroup, the shader-clock cycles
 *                (s_memtime) and the 100 MHz constant-clock ticks
 *                (s_memrealtime) of its first wave's MFMA loop; their ratio
 *                times 100 MHz is the shader clock under this load
 * Returns MXG_OK or an error status.
 */
#define MXG_CEIL_FP16 16
int mxgemm_mfma_ceiling(const void *ops, int64_t op_bytes, const uint8_t *scales,
                        int64_t scale_bytes, int kind, int64_t iters, int workgroups,
                        float *out, uint32_t *clocks, void *stream);

/*
 * mxgemm_device_supported - the hardware gate: 1 if the current HIP device is
 * gfx950 (the only target this library is built for; its scaled fp8/fp4
 * MFMA instructions exist nowhere else), 0 if not, a negative MXG_* status
 * if the runtime cannot be queried.  Every other entry point applies the same
 * check and returns MXG_EUNSUPPORTED instead of launching.  The RIGEL summary
 * ("Resumo Técnico: RIGEL", section "Contradições e Portões de Versão")
 * found its low-precision matrix formats present only behind a version gate
 * and binaries refusing to load elsewhere; here the gate is explicit and
 * queried at run time.  Thread-safe; the per-device answer is cached.
 */
int mxgemm_device_supported(void);

/*
 * mxgemm_status_string - static, NUL-terminated description of a status
 * code (never NULL; unknown codes get "unknown status").  Errors are
 * reported as a status plus no side effect, the convention of the WWDC26
 * session 330 summary, section "Scale Factor 付き量子化 tensor を作成する"
 * (a failed creation returns an error object and a nil tensor): a call that
 * returns nonzero has enqueued nothing and written nothing.
 */
const char *mxgemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MXGEMM_H */
