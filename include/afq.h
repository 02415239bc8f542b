/*
 * afq.h -- C ABI of the fused activation FP8 quantisation library
 *          (libafq.so, HIP kernels for AMD gfx950 / MI355X).
 *
 * The library quantises the input activation of an FP8 linear layer inside
 * the kernel that produces that activation, so the activation never makes a
 * bf16 round trip through HBM and no separate quant kernel is launched:
 *
 *   fused_add_rmsnorm_quant  residual add + RMSNorm (Gemma or standard),
 *                            one or two row segments per launch
 *   silu_mul_quant           SiLU-and-mul on a [gate | up] row
 *   swiglu_oai_quant         the clamped SwiGLU on a [gate | up] row
 *   fp8_quant                the standalone row-wise quantiser (the
 *                            "separate quant" the fused kernels replace)
 *
 * each emitting one of three quantised formats:
 *
 *   AFQ_MXFP8      1x32 blocks, one E8M0 byte per block, e4m3fn codes
 *                  (vLLM pull request 65478, MiniMax-M3.1 FFN MXFP8 quant
 *                  fusions, "Purpose"; scale layout: row-major [M, K/32],
 *                  not swizzled, as the review of that request and vLLM
 *                  pull request 65479 "AiterMxfp8LinearKernel" state for
 *                  the consuming GEMMs)
 *   AFQ_BLOCK128   1x128 groups, one fp32 scale amax/448 per group
 *                  (SGLang pull request 48043, "qwen3: Fuse the 1x128 FP8
 *                  input quant into RMSNorm and SiLU-and-mul", "Motivation"
 *                  and "Modifications")
 *   AFQ_PER_TOKEN  one fp32 scale amax/448 per row, shape [M, 1]
 *                  (SGLang pull request 34502, "Fuse per-token activation
 *                  quant into RMSNorm for per-channel quantized attention",
 *                  "Change")
 *
 * Arithmetic contract (what every entry point computes, per row):
 *   h   = round_dt(x + r)                       (only with a residual)
 *   y   = h * rsqrt(mean(h^2) + eps) * g        g = 1 + w (Gemma) or w
 *   u   = round_dt(y)                           the normed row; also the
 *                                               optional `normed` copy
 *   MXFP8:    b = max(expfield_fp32(amax|u|) - 8, 0)   (E8M0 byte)
 *             q = e4m3(clamp(u * 2^(127-b), -448, 448))
 *   1x128 / per-token:
 *             s = fp32(amax|u| / 448);  q = e4m3(clamp(fp32(u / s), +-448))
 *             (an all-zero group, and one whose amax / 448 rounds to zero
 *             in fp32 -- amax <= 224 * 2^-149, reachable from fp32 rows
 *             only -- stores s = 0 and codes 0x00)
 *   e4m3 rounding is round-to-nearest-even on OCP e4m3fn (max 448,
 *   subnormals k * 2^-9, sign in bit 7).
 * fp32-direct variant (quant_input = AFQ_QIN_FP32; 1x128 and per-token):
 *   the quantiser reads the fp32 normed value instead of its dtype rounding
 *   (the reading of AITER's fused 1x128 norm in SGLang pull request 48043,
 *   "Accuracy Tests"), in this order, every step rounded to fp32 once:
 *     inv32 = fl32(1 / sqrt(mean(h^2) + eps))  (mean(h^2) accumulated in fp64)
 *     y     = fl32(fl32(h * inv32) * g32)      g32 = fl32(1 + w) or w
 *     normed copy = round_dt(y);  s, q from y as above.
 * The norm itself is evaluated in fp32; the quantiser acts on the rounded
 * row u, so the result equals the unfused norm -> quant composition (vLLM
 * pull request 65478, "Test Plan / Correctness").
 *
 * SiLU-and-mul (silu_mul_quant), per element j of a row:
 *   MXFP8:    a_j = fp32(fp32(silu(gate_j)) * up_j) -- SiLU-and-mul in fp32
 *             arithmetic -- quantised without any bf16 rounding (vLLM pull
 *             request 65478, "Purpose", commit 2: the activation stays fp32
 *             between SiLU-and-mul and the quantiser).  The kernel's fp32
 *             silu is within 2 ulp of fp32(silu) for gates >= -80, and
 *             rounded to fp32 from an fp64 evaluation below.
 *   BLOCK128: a_j = bf16(bf16(silu(gate_j)) * up_j), the rounding of the
 *             unfused SiluAndMul, so the codes equal the unfused chain
 *             (SGLang pull request 48043, "Modifications")
 *   MXFP8 with quant_input = AFQ_QIN_BF16 (bf16-first variant): a_j is
 *             rounded to bf16 before the quantiser, as the unfused
 *             SiLU-and-mul -> quant chain stores it (vLLM pull request
 *             65478, "Test Plan / Correctness").
 *
 * Clamped SwiGLU (swiglu_oai_quant; MXFP8 only), per element j of a row:
 *   gc_j = min(gate_j, limit),  uc_j = min(max(up_j, -limit), limit)
 *   a_j  = fp32(fp32(gc_j * logistic(alpha * gc_j)) * fp32(uc_j + beta))
 *   quantised like the MXFP8 SiLU-and-mul (quant_input AFQ_QIN_BF16: a_j
 *   rounded to bf16 first).  vLLM pull request 65478 ("Microbenchmark
 *   script") times this activation as swiglu_oai(gu, 1.702, 1.0, 7.0) with a
 *   fused fp32 swiglu + MXFP8 kernel ("Purpose", commit 2); the pages do not
 *   write the function out, and the form above is the clamped SwiGLU
 *   published with OpenAI's gpt-oss models.  The kernel's fp32 gate factor
 *   is within a few ulp of fp32(gc * logistic(alpha * gc)).
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless stated otherwise; descriptors are
 *     host memory read during the call only.
 *   - The caller allocates and owns every buffer.  The library never
 *     allocates, frees, synchronises, or keeps a pointer after returning.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without waiting.  Calls are thread-safe and legal
 *     during stream capture (hipStreamBeginCapture); captured and eager
 *     launches compute bit-identical results.
 *   - Results are deterministic and batch-invariant: a row's outputs depend
 *     only on that row's inputs.
 *   - Every check except AFQ_ERR_LAUNCH is made on the host, before anything
 *     is enqueued; when a call returns an error nothing has been written.
 *     M == 0 returns AFQ_OK after the shape checks and enqueues nothing.
 *   - Overlap between buffers is judged on each buffer's byte span from its
 *     first to its last byte.
 *   - Inputs are assumed finite, and so is the rounded residual sum
 *     round_dt(x + r) (fp16 overflows above 65504); otherwise the outputs
 *     are unspecified (no error is reported and nothing outside the outputs
 *     is written).  The mean square is accumulated in fp32, so the same
 *     holds for rows whose sum of squares overflows fp32 (|h| above about
 *     1e19 / sqrt(cols)) and for mean(h^2) + eps == 0 (eps = 0 with an
 *     all-zero row); and, for SiLU-and-mul, for a quantisation group whose
 *     activation overflows its dtype (|silu(gate) * up| beyond the fp32 or
 *     bf16 range).
 *
 * Copy-only launches (ABI 3): when out.values and out.scales are both NULL
 * (in every segment of a norm launch), fused_add_rmsnorm_quant and
 * silu_mul_quant quantise nothing and write only the rounded activation
 * out.normed, which is then required (and, for the norm, the updated
 * residual).  These are the first kernels of the unfused chains: norm ->
 * fp8_quant and SiLU-and-mul -> fp8_quant, which the fused launches replace
 * (vLLM pull request 65478, "Kernel-level measurements": the "norm +
 * separate quant" and "swiglu + separate quant" columns).  The copy is the
 * same as a quantising launch's copy: u for the norm (any mode), and for
 * SiLU-and-mul the activation rounded to bf16 as `mode` rounds it (MXFP8:
 * bf16(a) of the fp32 activation; BLOCK128: bf16(bf16(silu) * up)).  Widths
 * need only be multiples of 8; quant_input must be AFQ_QIN_DEFAULT
 * (otherwise AFQ_ERR_UNSUPPORTED).  Only one of values / scales being NULL
 * is AFQ_ERR_NULL.
 */
#ifndef AFQ_H
#define AFQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AFQ_ABI_VERSION 4

/* Return codes. */
enum {
    AFQ_OK = 0,
    AFQ_ERR_NULL = -1,        /* a required pointer (or the descriptor) is NULL */
    AFQ_ERR_SHAPE = -2,       /* M < 0 or above AFQ_MAX_ROWS, cols/I not a positive
                                 multiple of the group size and of 8, cols above
                                 AFQ_MAX_COLS, row stride smaller than the row or
                                 above AFQ_MAX_ROW_STRIDE, a buffer that would run
                                 past the end of the address space, nseg not 1 or 2,
                                 or a residual with two segments */
    AFQ_ERR_ALIGN = -3,       /* a base pointer or row pitch not 16-byte aligned
                                 (scales: 4-byte aligned) */
    AFQ_ERR_DTYPE = -4,       /* dtype not allowed for this entry point */
    AFQ_ERR_ALIAS = -5,       /* an output overlaps another output or an input
                                 (residual_out == residual_in is allowed) */
    AFQ_ERR_UNSUPPORTED = -6, /* mode, kind or quant_input not offered by this
                                 entry point (for this mode) */
    AFQ_ERR_ARG = -7,         /* eps negative or not finite, unknown enum value
                                 (quant_input included) */
    AFQ_ERR_LAUNCH = -8       /* the HIP launch failed; see afq_last_hip_error() */
};

/* Quantisation modes. */
enum { AFQ_MXFP8 = 0, AFQ_BLOCK128 = 1, AFQ_PER_TOKEN = 2 };
/* Activation dtypes. */
enum { AFQ_BF16 = 0, AFQ_FP16 = 1, AFQ_FP32 = 2 };
/* RMSNorm kinds: y = n * w (standard) or y = n * (1 + w) (Gemma). */
enum { AFQ_RMSNORM_STANDARD = 0, AFQ_RMSNORM_GEMMA = 1 };
/* What the quantiser reads (afq_norm_desc / afq_act_desc .quant_input).
 *   AFQ_QIN_DEFAULT  norm: the dtype-rounded normed row (every mode);
 *                    SiLU: MXFP8 the fp32 activation, 1x128 the bf16 one
 *   AFQ_QIN_FP32     norm, AFQ_BLOCK128 and AFQ_PER_TOKEN only: the fp32
 *                    normed value (fp32-direct)
 *   AFQ_QIN_BF16     SiLU, AFQ_MXFP8 only: the fp32 activation rounded to
 *                    bf16 (bf16-first)
 * Another value is AFQ_ERR_ARG; a value another path or mode does not
 * offer is AFQ_ERR_UNSUPPORTED. */
enum { AFQ_QIN_DEFAULT = 0, AFQ_QIN_FP32 = 1, AFQ_QIN_BF16 = 2 };

/* Largest row width (per segment) the kernels are built for. */
#define AFQ_MAX_COLS 32768
/* Largest row count of one call (the row kernels launch up to one
 * workgroup per row). */
#define AFQ_MAX_ROWS 2147483647
/* Largest row stride, in elements. */
#define AFQ_MAX_ROW_STRIDE ((int64_t)1 << 40)

/*
 * A quantised activation (the tuple a quantised linear consumes: codes,
 * scales, and optionally the activation rounded to its dtype).
 *   values  e4m3fn codes, [rows, cols] dense row-major.  Required, unless
 *           values and scales are both NULL (a copy-only launch).
 *   scales  MXFP8: uint8 E8M0 [rows, cols/32]; BLOCK128: float
 *           [rows, cols/128]; PER_TOKEN: float [rows, 1].  Dense
 *           row-major, unswizzled.  Required as values is; 4-byte aligned.
 *   normed  [rows, cols] dense copy of the rounded activation in the
 *           activation dtype (the norm output u, or for SiLU-and-mul the
 *           bf16 activation); NULL = not written.  Required by a copy-only
 *           launch.
 * The tags that the pages' quantised-activation tuples carry beside codes
 * and scales -- the mode, the original dtype and shape (vLLM pull request
 * 65479, QuantizedActivation; SGLang pull request 34502, "Change") -- are
 * not repeated here: the caller owns this struct and has just passed each
 * of them in the descriptor (mode, dtype, M and cols), and the library
 * writes nothing but device buffers.  The Python binding's result object
 * carries them.
 */
typedef struct afq_qact {
    void *values;
    void *scales;
    void *normed;
} afq_qact;

/* One row segment of a norm launch. */
typedef struct afq_norm_seg {
    const void *x;        /* [M, cols] in dtype, row pitch x_row_stride elements */
    int64_t x_row_stride; /* elements, >= cols; pitch in bytes a multiple of 16 */
    const void *weight;   /* [cols] in dtype */
    int64_t cols;         /* row width of this segment */
    afq_qact out;
} afq_norm_seg;

/*
 * fused_add_rmsnorm_quant descriptor.
 *   M            rows (>= 0)
 *   quant_input  AFQ_QIN_DEFAULT, or AFQ_QIN_FP32 (1x128 / per-token)
 *   nseg         1, or 2 for two independent row segments normed in one
 *                launch with separate weights (the q / kv RMSNorm of MLA
 *                attention: SGLang pull request 34502, "Change", decode
 *                q_b_proj site).  Each segment has its own scales.
 *   kind, dtype  afq_norm_kind; AFQ_BF16 or AFQ_FP16 (inputs, weight,
 *                residual and normed copy all share dtype)
 *   mode         afq_quant_mode
 *   eps          added to the mean square; finite and >= 0
 *   residual_in  [M, cols] dense, or NULL for a plain RMSNorm (h = x).
 *                Only with nseg == 1.
 *   residual_out [M, cols] dense, receives h = round_dt(x + residual_in);
 *                must be non-NULL exactly when residual_in is; may equal
 *                residual_in (in-place update of the residual stream).
 */
typedef struct afq_norm_desc {
    int64_t M;
    int32_t nseg;
    int32_t kind;
    int32_t dtype;
    int32_t mode;
    float eps;
    int32_t quant_input; /* AFQ_QIN_DEFAULT or AFQ_QIN_FP32 */
    const void *residual_in;
    void *residual_out;
    afq_norm_seg seg[2];
} afq_norm_desc;

/*
 * silu_mul_quant descriptor.
 *   M, I           rows, and width of the activation (the input row is 2I)
 *   gate_up        bf16 [M, 2I]: gate = columns [0, I), up = [I, 2I)
 *   gate_up_row_stride  elements, >= 2I; pitch in bytes a multiple of 16
 *   mode           AFQ_MXFP8 or AFQ_BLOCK128 (AFQ_PER_TOKEN is not offered:
 *                  AFQ_ERR_UNSUPPORTED)
 *   quant_input    AFQ_QIN_DEFAULT, or AFQ_QIN_BF16 (MXFP8)
 *   out            [M, I] codes and scales; out.normed = optional bf16 copy
 *                  of the activation a.
 */
typedef struct afq_act_desc {
    int64_t M;
    int64_t I;
    const void *gate_up;
    int64_t gate_up_row_stride;
    int32_t mode;
    int32_t quant_input; /* AFQ_QIN_DEFAULT or AFQ_QIN_BF16 */
    afq_qact out;
} afq_act_desc;

/*
 * swiglu_oai_quant descriptor (ABI 4).
 *   act     rows, width, input, quant_input and outputs exactly as for
 *           silu_mul_quant; act.mode must be AFQ_MXFP8 (otherwise
 *           AFQ_ERR_UNSUPPORTED).  A copy-only launch (values and scales
 *           NULL) writes the bf16 activation bf16(a_j).
 *   alpha   slope of the logistic gate; finite
 *   beta    added to the clamped up value; finite
 *   limit   clamp bound; > 0, +inf allowed (no clamping)
 * Bad alpha, beta or limit: AFQ_ERR_ARG.
 */
typedef struct afq_swiglu_desc {
    afq_act_desc act;
    float alpha;
    float beta;
    float limit;
} afq_swiglu_desc;

/*
 * fp8_quant descriptor: the standalone quantiser of an activation that is
 * already in HBM (the "separate quant" of the unfused chains: vLLM pull
 * request 65478 mxfp8_e4m3_quantize, "Kernel-level measurements"; SGLang
 * pull request 48043 per-1x128 quant; SGLang pull request 34502 per-token
 * quant).
 *   x        [M, cols] in dtype (AFQ_BF16, AFQ_FP16 or AFQ_FP32), row pitch
 *            x_row_stride elements (pitch in bytes a multiple of 16)
 *   out      codes and scales; out.normed must be NULL.
 */
typedef struct afq_quant_desc {
    int64_t M;
    int64_t cols;
    const void *x;
    int64_t x_row_stride;
    int32_t dtype;
    int32_t mode;
    afq_qact out;
} afq_quant_desc;

/* Residual add + RMSNorm + quantisation.  Returns AFQ_OK or an AFQ_ERR_*. */
int fused_add_rmsnorm_quant(const afq_norm_desc *desc, void *stream);

/* SiLU-and-mul + quantisation.  Returns AFQ_OK or an AFQ_ERR_*. */
int silu_mul_quant(const afq_act_desc *desc, void *stream);

/* Clamped SwiGLU + MXFP8 quantisation.  Returns AFQ_OK or an AFQ_ERR_*. */
int swiglu_oai_quant(const afq_swiglu_desc *desc, void *stream);

/* Standalone row-wise quantisation.  Returns AFQ_OK or an AFQ_ERR_*. */
int fp8_quant(const afq_quant_desc *desc, void *stream);

/* Static English text for a return code (never NULL). */
const char *afq_status_string(int status);

/* AFQ_ABI_VERSION of the loaded library. */
int afq_abi_version(void);

/* The hipError_t behind the calling thread's last AFQ_ERR_LAUNCH (0 if none). */
int afq_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* AFQ_H */
