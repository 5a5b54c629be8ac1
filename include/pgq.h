/*
 * pgq.h -- per-row symmetric weight quantization on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpgq.so.  Plain pointers and sizes only.  Every data pointer below is a
 * DEVICE pointer on the current HIP device unless the comment says "host".  `stream`
 * is a hipStream_t passed as void* (NULL = the default stream).  All calls are
 * asynchronous on `stream`; none synchronizes it.
 *
 * What is computed (Parameter Golf submission pages):
 *   - per-row quantization, percentile clipping for export and small-tensor FP16
 *     passthrough: "Swiglu gating ... 10min/16MB Track" (PR #2159), list "Key Explored
 *     Modifications";
 *   - 6-bit codes in [-31, 31] and STE fake quantization in the forward pass: "SubSixteen
 *     v2: Int6 QAT + MLP 3x + SWA" card (PR #69), sections Quantization and Other;
 *   - int8 for the tensors named by QUANT_INT8_NAME_PATTERNS (default tok_emb.weight,
 *     lm_head.weight) and int6 AWQ export: "12L 24min Vocab1792 ... Int6AWQ MixedBits"
 *     (PR #1495), Submission summary and Mixed-bit quantization details;
 *   - averaging of quantize-dequantize snapshots (SQWA): "Discriminative TTT + SLOT-24"
 *     card (PR #1414), Novel Contributions;
 *   - EMA of the weights (decay 0.997): PR #1414 and "Unified Attention + FA3 + Legal TTT"
 *     (PR #1202) cards, Weight Averaging; SWA over checkpoints: PR #69 card, Novel
 *     Contributions and Weight Averaging;
 *   - per-tensor scales: PR #2159 list (per-row / per-tensor quantization strategy);
 *   - 6-bit code storage and its decode: the int6 artifact savings of the PR #69 card (the
 *     byte layout is this library's own, documented at pgq_dequant_codes);
 *   - the forward matmul over the STE-dequantized weights, dequantization fused: PR #69
 *     card, section Other.
 *
 * The arithmetic, fixed where the pages leave it open (Q = 2^(bits-1) - 1, every step an
 * IEEE binary32 operation with round-to-nearest-even):
 *   x_j   = w_j                         (AWQ: x_j = w_j * a_j,  a_j = fp16(sqrt(s_j)))
 *   clip  = k-th smallest |x_j|, k = ceil(pct_num * n / pct_den) clamped to [1, n]
 *   s     = fp16(clip / Q); s = 1.0 when that rounds to zero
 *   t_j   = x_j / s;  code_j = clamp(rne(t_j), -Q, Q)
 *   dq_j  = code_j * s                  (AWQ: dq_j = (code_j * s) / a_j)
 *   STE:  mask_j = |t_j| <= Q + 1/2;  grad_out_j = mask_j ? grad_j : +0
 *   SQWA: mean = xhat (k = 1), mean = mean + (xhat - mean) / k (k > 1)
 *
 * Errors.  Argument errors return a pgq_status synchronously and enqueue nothing.
 * Conditions that depend on the data (NaN/Inf inputs, scale or fp16 overflow, bad AWQ
 * scales, a stale descriptor table) are OR-ed into *dev_status on the device with an
 * atomic; the library never clears that word.  Outputs of an affected row are
 * unspecified.
 *
 * Ownership.  The caller allocates every device buffer and keeps it alive until the
 * stream work that uses it has completed.  The library allocates no device memory and
 * keeps no state besides a per-device cache of launch limits; it is thread-safe.  Host
 * arrays are read during the call only.  Inputs and outputs must not overlap, except
 * that `mean` is updated in place.
 */
#ifndef PGQ_H
#define PGQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PGQ_OK = 0,
    PGQ_ERR_NULL = 1,       /* a required pointer is NULL */
    PGQ_ERR_SHAPE = 2,      /* negative size, ld < cols, too many rows */
    PGQ_ERR_DTYPE = 3,      /* unsupported element type for this call */
    PGQ_ERR_PARAM = 4,      /* bits outside [2, 8], pct_den == 0 or pct_num > pct_den, bad mode/k/kind */
    PGQ_ERR_ALIGN = 5,      /* pointer not aligned to its element size */
    PGQ_ERR_WORKSPACE = 6,  /* workspace missing or smaller than required */
    PGQ_ERR_HIP = 7         /* a HIP runtime call or kernel launch failed */
} pgq_status;

/* Bits OR-ed into *dev_status by the kernels. */
#define PGQ_DEV_NONFINITE   1u   /* a NaN or infinity in an input row */
#define PGQ_DEV_SCALE_OVF   2u   /* clip / Q rounds to fp16 infinity (clip >= 65520 * Q) */
#define PGQ_DEV_F16_OVF     4u   /* an fp16 passthrough value rounded to infinity */
#define PGQ_DEV_BAD_AWQ     8u   /* an AWQ activation scale is <= 0 or not finite */
#define PGQ_DEV_STALE_TABLE 16u  /* PGQ_TABLE_RESIDENT given but the workspace holds another table; nothing was written */

/* Element types.  Weight inputs may be any of the three; dequantized outputs PGQ_F32 or
 * PGQ_BF16.  fp16 weights are widened to binary32 exactly before every step. */
#define PGQ_F32  0
#define PGQ_BF16 1
#define PGQ_F16  2

/* Export kinds: an integer kind is its bit width; PGQ_KIND_F16 is fp16 passthrough. */
#define PGQ_KIND_F16 16

/* Flags for the grouped calls. */
#define PGQ_TABLE_RESIDENT 1u    /* the workspace already holds the descriptor table that an earlier
                                    call of the same entry point wrote for identical arguments: skip
                                    the upload.  The kernels compare a checksum of the table with the
                                    one this call computes and write nothing if they differ
                                    (PGQ_DEV_STALE_TABLE). */

/* Quantizer parameters: code width and the clip percentile pct_num / pct_den
 * (1/1 = absolute maximum; 9999/10000 = 99.99th percentile). */
typedef struct {
    int32_t bits;       /* 2..8; Q = 2^(bits-1) - 1 (6 -> 31, 8 -> 127) */
    uint32_t pct_num;   /* 0 <= pct_num <= pct_den */
    uint32_t pct_den;   /* > 0 */
} pgq_qparams;

/* ------------------------------------------------------------------------------------------ */
/* One matrix.                                                                                  */
/* ------------------------------------------------------------------------------------------ */

/* Quantize each row of a rows x cols matrix (row stride ld elements, ld >= cols).
 *   w         input, PGQ_F32, PGQ_BF16 or PGQ_F16 (w_dtype)
 *   awq_s     NULL, or cols fp32 activation scales s_j > 0: the row is multiplied by
 *             a_j = fp16(sqrt(s_j)) before quantization and divided by it in dequant
 *   awq_mult  NULL, or cols fp16 outputs (bit patterns) receiving a_j
 *   codes     NULL, or rows x cols int8 codes (row stride cols)
 *   scales    rows fp16 scales (bit patterns); required
 *   dq        NULL, or rows x cols dequantized values (row stride cols) of type dq_dtype
 * Source: per-row quantization and percentile clipping (PR #2159, Key Explored
 * Modifications); range [-31, 31] for 6 bits (PR #69 card, section Other); int6 AWQ
 * export (PR #1495, Submission summary). */
pgq_status pgq_quantize_rows(const void* w, int32_t w_dtype, int64_t rows, int64_t cols, int64_t ld,
                             pgq_qparams qp, const float* awq_s, uint16_t* awq_mult,
                             int8_t* codes, uint16_t* scales, void* dq, int32_t dq_dtype,
                             uint32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------------------------ */
/* STE fake quantization for quantization-aware training (grouped over n bf16 matrices).       */
/* Source: PR #69 card, section Other (straight-through estimator fake quantization in the     */
/* forward pass, range [-31, 31]) and section Quantization (STE QAT, 6 bits).                  */
/* ------------------------------------------------------------------------------------------ */

#define PGQ_FQ_FWD     1   /* w -> dq, scales, mask (and codes) */
#define PGQ_FQ_BWD     2   /* mask, grad -> grad_out */
#define PGQ_FQ_FWD_BWD 3   /* both, in one pass over w and grad */

typedef struct {
    const uint16_t* w;      /* bf16 weights, rows x cols, row stride ld (FWD, FWD_BWD) */
    int64_t rows, cols, ld;
    uint16_t* dq;           /* bf16 fp32->bf16(code * s), rows x cols dense (FWD, FWD_BWD) */
    uint16_t* scales;       /* fp16, rows (FWD, FWD_BWD) */
    uint8_t* mask;          /* rows x ceil(cols/8) bytes, bit j%8 of byte j/8 = mask_j.  Written by
                               FWD and FWD_BWD (may be NULL there), read by BWD */
    const uint16_t* grad;   /* bf16 upstream gradient, rows x cols dense (BWD, FWD_BWD) */
    uint16_t* grad_out;     /* bf16 masked gradient, rows x cols dense (BWD, FWD_BWD) */
    int8_t* codes;          /* NULL or rows x cols int8 codes (FWD, FWD_BWD) */
} pgq_fq_tensor;

/* Workspace bytes the grouped fake-quant call needs for these n tensors. */
pgq_status pgq_fakequant_workspace(const pgq_fq_tensor* t, int32_t n, size_t* workspace_bytes);

/* mode: PGQ_FQ_*.  t: host array of n descriptors.  workspace: device scratch of at least
 * pgq_fakequant_workspace() bytes (may be NULL when n == 1).  flags: 0 or PGQ_TABLE_RESIDENT. */
pgq_status pgq_fakequant_fwd_bwd(int32_t mode, const pgq_fq_tensor* t, int32_t n, pgq_qparams qp,
                                 void* workspace, size_t workspace_bytes, uint32_t flags,
                                 uint32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------------------------ */
/* Whole-model export (one grouped launch over every tensor).                                  */
/* Source: PR #2159 Key Explored Modifications (per-row quantization, percentile clipping,     */
/* small-tensor FP16 passthrough); PR #1495 Mixed-bit quantization details (int6 by default,   */
/* int8 for names matching QUANT_INT8_NAME_PATTERNS) and Submission summary (int6 AWQ).        */
/* ------------------------------------------------------------------------------------------ */

typedef struct {
    const char* name;       /* host string used by the policy (NULL = "") */
    const void* w;          /* device input, rows x cols, row stride ld */
    int32_t dtype;          /* PGQ_F32, PGQ_BF16 or PGQ_F16 */
    int32_t reserved;
    int64_t rows, cols, ld; /* 1-D tensors: rows = 1; higher ranks: rows = shape[0] */
    const float* awq_s;     /* NULL or cols fp32 activation scales (used for integer kinds whose
                               bits equal the policy's default bits) */
} pgq_tensor_in;

typedef struct {
    const char* const* int8_patterns; /* host array of n_patterns host strings; a tensor whose name
                                         contains one of them (substring) uses q_sensitive */
    int32_t n_patterns;
    int32_t per_tensor;               /* 0: one scale per row; 1: one scale per integer-kind tensor,
                                         its clip the percentile of |w| over the whole tensor
                                         (PR #2159 Key Explored Modifications: per-row / per-tensor
                                         quantization, percentile clipping).  Not with AWQ. */
    int64_t passthrough_below;        /* tensors with fewer elements are stored as fp16 (65536) */
    pgq_qparams q_default;            /* e.g. {6, 9999, 10000} */
    pgq_qparams q_sensitive;          /* e.g. {8, 1, 1} */
    int32_t pack6;                    /* 1: 6-bit tensors store their codes four per three bytes
                                         (the int6 artifact savings of the PR #69 card; layout
                                         below at pgq_dequant_codes) */
    int32_t reserved;
} pgq_policy;

typedef struct {
    int32_t kind;           /* PGQ_KIND_F16, or the code width in bits */
    int32_t has_awq;        /* 1 when AWQ multipliers are produced for this tensor */
    pgq_qparams qp;         /* quantizer of an integer kind */
    int32_t per_tensor;     /* 1: one scale for the whole tensor (scales region holds 1 fp16) */
    int64_t codes_off;      /* byte offsets into the arena; -1 when absent */
    int64_t scales_off;
    int64_t f16_off;
    int64_t awq_off;
    int32_t packed;         /* 1: codes region holds 6-bit packed codes, 3 * ceil(cols / 4) bytes per row */
    int32_t reserved;
} pgq_tensor_plan;

/* Host only (no device work): decide each tensor's kind and lay out the output arena.
 * plan: host array of n entries (written).  arena_bytes / workspace_bytes: sizes the
 * caller must allocate for pgq_export_model / pgq_sqwa_accumulate.  Regions are 256-byte
 * aligned: codes rows x cols int8 (packed: rows x 3 * ceil(cols / 4) bytes), scales rows fp16
 * (1 when per_tensor), f16 numel fp16, awq cols fp16.  PGQ_ERR_PARAM when per_tensor meets AWQ scales; PGQ_ERR_SHAPE when a per-tensor
 * tensor has 2^32 elements or more. */
pgq_status pgq_export_plan(const pgq_tensor_in* t, int32_t n, const pgq_policy* pol,
                           pgq_tensor_plan* plan, size_t* arena_bytes, size_t* workspace_bytes);

/* Quantize every tensor into the arena in one launch.  dq_out: NULL, or a host array of n
 * device pointers (each NULL or rows x cols fp32) receiving the value each tensor decodes to
 * (code * s, AWQ-divided, or fp32(fp16) for passthrough).  With per-tensor entries the launch
 * is preceded by the whole-tensor clip select: one pass for an absmax clip, else four radix
 * passes, each one launch over those tensors (their select state lives in the workspace).
 * After an error return, call again without PGQ_TABLE_RESIDENT. */
pgq_status pgq_export_model(const pgq_tensor_in* t, int32_t n, const pgq_tensor_plan* plan,
                            void* arena, float* const* dq_out, void* workspace, size_t workspace_bytes,
                            uint32_t flags, uint32_t* dev_status, void* stream);

/* The same export for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): no workspace argument; the descriptor
 * table and the whole-tensor select state live in a 4 MiB array of device memory that the library
 * holds for each GPU it runs on until the process ends.  Nothing is allocated or freed by the call.
 * Returns PGQ_ERR_WORKSPACE (nothing enqueued) when the call's table needs more than 4 MiB (the
 * workspace_bytes pgq_export_plan reports is that size).  Every call on one GPU shares its array,
 * which keeps the last call's table: calls that overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller.  PGQ_TABLE_RESIDENT skips the upload when the
 * array still holds this call's table (checked by checksum, as for pgq_export_model). */
pgq_status pgq_export_model_noalloc(const pgq_tensor_in* t, int32_t n, const pgq_tensor_plan* plan, void* arena,
                                    float* const* dq_out, uint32_t flags, uint32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------------------------ */
/* SQWA: fold snapshot k (1-based) into per-tensor fp32 running means.                         */
/* Source: "Discriminative TTT + SLOT-24" card (PR #1414), Novel Contributions: average        */
/* quantize-dequantize snapshots.  Each snapshot tensor is quantized and dequantized with the  */
/* plan's kind (fp16 round trip for passthrough), then mean = xhat (k = 1) or                  */
/* mean + (xhat - mean) / k.  Export the final mean with pgq_export_model and the same plan.   */
/* ------------------------------------------------------------------------------------------ */
pgq_status pgq_sqwa_accumulate(const pgq_tensor_in* snap, int32_t n, const pgq_tensor_plan* plan,
                               float* const* mean, int32_t k, void* workspace, size_t workspace_bytes,
                               uint32_t flags, uint32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------------------------ */
/* Decode stored codes back to fp32 weights (the artifact loader): x = code * s, divided by     */
/* a_j when awq_mult is given -- bit for bit the dequantized value the export produced.        */
/* Source: the int6 artifact savings of the "SubSixteen v2" card (PR #69), Novel              */
/* Contributions; the pages give no byte layout, so the 6-bit layout below is ours.           */
/*   codes      device, rows x cols int8 (packed = 0) or rows x 3 * ceil(cols / 4) bytes        */
/*              (packed = 1): per row, group g of three bytes is the little-endian 24-bit word  */
/*              holding codes 4g .. 4g+3 as 6-bit two's complement fields, code 4g + t in bits  */
/*              6t .. 6t+5; a short last group is padded with code 0                            */
/*   scales     device fp16 bit patterns: rows of them, or one when per_tensor = 1              */
/*   awq_mult   NULL, or device cols fp16 multipliers a_j (bit patterns, as exported)           */
/*   out        device rows x cols fp32, dense                                                  */
/* Reads and writes only; no status bits are produced (dev_status may be NULL).                */
/* ------------------------------------------------------------------------------------------ */
pgq_status pgq_dequant_codes(const void* codes, int32_t packed, int64_t rows, int64_t cols, const uint16_t* scales,
                             int32_t per_tensor, const uint16_t* awq_mult, float* out, uint32_t* dev_status,
                             void* stream);

/* The whole exported model back to fp32 in one grouped launch: for each tensor i with out[i]  */
/* non-NULL (fp32 rows x cols dense), the decode above of its arena regions (plan[i] as        */
/* pgq_export_plan wrote it), or fp32 of the stored fp16 values for passthrough tensors.      */
/* t supplies the shapes only (w and name are ignored).  workspace: at least the              */
/* workspace_bytes pgq_export_plan reported (descriptor table; PGQ_TABLE_RESIDENT as usual). */
pgq_status pgq_dequant_model(const pgq_tensor_in* t, int32_t n, const pgq_tensor_plan* plan, const void* arena,
                             float* const* out, void* workspace, size_t workspace_bytes, uint32_t flags,
                             uint32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------------------------ */
/* The QAT forward's consumer GEMM with the STE dequantization fused in.  Source: "SubSixteen   */
/* v2" card (PR #69), section Other: STE fake quantization in the forward pass -- the layer's  */
/* matmul consumes What[n][k] = bf16(fp32(code[n][k] * s_n)), which this call forms on the fly  */
/* from the codes and scales instead of reading a materialised bf16 weight.                    */
/*   Y[m][n] = sum_k X[m][k] * What[n][k], accumulated in fp32 on the matrix cores (MFMA)      */
/*   x       device bf16 bit patterns, M x K, row stride ldx >= K                              */
/*   codes   device int8, N x K, row stride ldc >= K (e.g. the fake-quant call's codes output)  */
/*   scales  device fp16 bit patterns, N (one per weight row)                                   */
/*   y       device fp32, M x N, row stride ldy >= N (written, not accumulated into)           */
/* M <= 65535 * 128.  K = 0 writes zeros.  Asynchronous on stream.                             */
pgq_status pgq_qgemm_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* codes, int64_t ldc,
                          const uint16_t* scales, int64_t N, float* y, int64_t ldy, void* stream);

/* The same GEMM with Y stored as bf16: the QAT forward's activations are bf16 (same card and    */
/* section).  Every element is bf16 (round to nearest even) of the fp32 value pgq_qgemm_bf16    */
/* writes for the same inputs, bit for bit: the accumulation is shared, only the store differs. */
/*   y       device bf16 bit patterns, M x N, row stride ldy >= N (written, not accumulated)    */
/* Other arguments, limits and errors as for pgq_qgemm_bf16; y must be 2-byte aligned.         */
pgq_status pgq_qgemm_bf16_ybf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* codes,
                                int64_t ldc, const uint16_t* scales, int64_t N, uint16_t* y, int64_t ldy, void* stream);

/* ------------------------------------------------------------------------------------------ */
/* Weight averaging without quantization, grouped over n tensors in one launch.               */
/* w[i]: the weights (fp32 or bf16, rows x cols, row stride ld; awq_s must be NULL; name is    */
/* ignored).  The averages are caller-owned fp32 device buffers, rows x cols dense, updated in */
/* place.  workspace: device memory of at least pgq_average_workspace() bytes, 64-byte aligned, */
/* holding the descriptor table (flags: PGQ_TABLE_RESIDENT as for the other grouped calls).   */
/* dev_status gets PGQ_DEV_NONFINITE when a weight or an updated average is NaN or infinite.  */
/* ------------------------------------------------------------------------------------------ */
pgq_status pgq_average_workspace(const pgq_tensor_in* w, int32_t n, size_t* workspace_bytes);

/* EMA.  Source: "Discriminative TTT + SLOT-24" (PR #1414) and PR #1202 cards, section Weight   */
/* Averaging: EMA with decay 0.997.  ema = fp32(fp32(decay * ema) + fp32(c * w)) with          */
/* c = fp32(1 - decay) (binary32, no fused multiply-add); init != 0 sets ema = w instead.     */
/* decay must lie in [0, 1] (PGQ_ERR_PARAM otherwise).                                        */
pgq_status pgq_ema_update(const pgq_tensor_in* w, int32_t n, float* const* ema, float decay, int32_t init,
                          void* workspace, size_t workspace_bytes, uint32_t flags, uint32_t* dev_status,
                          void* stream);

/* SWA.  Source: "SubSixteen v2" card (PR #69), Novel Contributions and Weight Averaging:      */
/* stochastic weight averaging over 16 checkpoints.  Fold checkpoint k (1-based, k <= 2^24)    */
/* into the running mean: mean = w (k = 1), else fp32(mean + fp32(fp32(w - mean) / k)) -- the  */
/* SQWA update applied to the weights themselves.  Which steps are checkpoints is the caller's. */
pgq_status pgq_swa_accumulate(const pgq_tensor_in* w, int32_t n, float* const* mean, int32_t k, void* workspace,
                              size_t workspace_bytes, uint32_t flags, uint32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------------------------ */
/* Timing aid (no method step): the next pgq_* call made by this host thread that launches     */
/* kernels records start_event when its first kernel begins executing and stop_event when its */
/* last kernel completes, from the kernels' own dispatches (hipExtLaunchKernel), so the pair   */
/* times the call's kernels alone.  The events are hipEvent_t handles passed as void* (created */
/* by the caller, not owned); NULL, NULL clears a pending request.  Applies to one call.       */
/* ------------------------------------------------------------------------------------------ */
pgq_status pgq_time_next_launch(void* start_event, void* stop_event);

/* ------------------------------------------------------------------------------------------ */
const char* pgq_status_str(pgq_status s);   /* static string */
const char* pgq_version(void);              /* static string */
/* Text of the HIP runtime error behind the calling thread's most recent PGQ_ERR_HIP ("" if     */
/* there was none); a static string owned by the HIP runtime.                                   */
const char* pgq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PGQ_H */
