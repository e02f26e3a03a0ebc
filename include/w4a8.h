/*
 * w4a8.h -- C ABI of libw4a8: a W4A8 quantized linear layer for AMD Instinct
 * MI355X (gfx950).
 *
 *   Y[M,N] (fp16) = X[M,K] . W[N,K]^T
 *
 * Weights are quantized offline in two levels (per-output-channel symmetric
 * INT8 in the protective range [-119, 119] with an fp16 scale s0, then per
 * group of 128 consecutive k asymmetric UINT4 with an integer scale s1 and a
 * zero point z).  Activations are quantized per token to INT8 by their
 * absolute maximum.  The GEMM main loop rebuilds INT8 weights in registers as
 * q4*s1 - z*s1 and contracts them with the INT8 activations on the INT8 matrix
 * cores into INT32; an fp32 epilogue applies s_a[m] and s0[n] and writes fp16.
 *
 * Pages the operations follow (by title and section):
 *  - QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM
 *    Serving (talk summary): "Progressive Group Quantization for W4A8 GEMM",
 *    "Precision Data Flow and Activation Quantization Fusion", "Quantized
 *    Matrix Multiplication (GEMM) Kernel on GPUs", "Challenges and Design
 *    Details of QServe GEMM Kernel".
 *  - Lecture 15 notes: 15.5 (dequantization inside the main loop) and 15.6
 *    (two-level quantization, int4 -> int8 by one multiply and one subtract).
 *  - QFactory reading notes: 2.1 (asymmetric quantization, w = (q - zero) * scale).
 *
 * Conventions for every entry point:
 *  - Ownership: every buffer argument is device memory allocated and freed by
 *    the caller (unless marked "host").  The library never allocates, frees
 *    or keeps per-call state; it is safe to call from several host threads.
 *  - Streams: all device work is enqueued on `stream` (0 = the null stream)
 *    and is asynchronous; results are ready when the stream is synchronised.
 *  - Alignment: device pointers must be 16-byte aligned.
 *  - Errors: argument errors (W4A8_E_NULL, W4A8_E_SHAPE, W4A8_E_ALIGN,
 *    W4A8_E_WORKSPACE) are detected on the host before anything is launched
 *    and leave every buffer untouched.  W4A8_E_HIP reports a launch failure
 *    (hipGetLastError after the launch).  No C++ exception crosses the ABI.
 *  - Shapes: K > 0 and K % 128 == 0; N > 0 and N % 16 == 0; M >= 0.  M == 0
 *    is a successful no-op.  Inputs must be finite; the results for NaN or
 *    Inf inputs are unspecified.  The GEMM entry points also need
 *    K <= 2^22 (W4A8_E_SHAPE otherwise).
 *  - Results are deterministic: bit-identical from run to run.
 */
#ifndef W4A8_H
#define W4A8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum w4a8_status {
    W4A8_OK = 0,
    W4A8_E_NULL = -1,       /* a required pointer is NULL                  */
    W4A8_E_SHAPE = -2,      /* M < 0, N <= 0, K <= 0, K % 128, N % 16, ld  */
    W4A8_E_ALIGN = -3,      /* a device pointer is not 16-byte aligned      */
    W4A8_E_WORKSPACE = -4,  /* workspace smaller than required              */
    W4A8_E_HIP = -5,        /* a HIP launch or runtime call failed          */
    W4A8_E_SCRATCH = -6     /* gemm_w4a8_noalloc: workspace need > scratch  */
} w4a8_status;

/* Text for a status code (host; static storage, never NULL). */
const char *w4a8_status_string(w4a8_status st);

/* Library version as "major.minor.patch" (host; static storage). */
const char *w4a8_version(void);

/* ------------------------------------------------------------------------
 * Offline weight quantization (QServe talk summary, "Progressive Group
 * Quantization for W4A8 GEMM"; Lecture 15 notes, 15.6).
 * ------------------------------------------------------------------------ */

/* Bytes of the device weight stream for an N x K weight (host).  Returns 0
 * for an invalid shape.  The stream holds the packed UINT4 codes (N*K/2
 * bytes) followed by one byte of group parameters per (n, group)
 * ((s1 - 1) | z << 4); its internal order is private to the library. */
size_t w4a8_packed_weight_bytes(int64_t N, int64_t K);

/* Quantize fp32 weights w [N, K] (row-major, row stride K) in two levels.
 *   level 1, per output channel n:
 *     s0[n] = fp16_rne(max_k |w[n,k]| / 119)   (fp32 division)
 *     q8    = clamp(rint(w / float(s0[n])), -119, 119)   (0 if s0 == 0)
 *   level 2, per group j of 128 consecutive k in row n (integers):
 *     lo = min(0, min q8), hi = max(0, max q8)
 *     s1 = max(1, ceil((hi - lo) / 15))  in [1, 16]
 *     z  = rne(-lo / s1)                 in [0, 15]
 *     q4 = clamp(rne(q8 / s1) + z, 0, 15)
 * Writes the device weight stream `wpacked` (w4a8_packed_weight_bytes(N, K)
 * bytes) and s0_fp16 [N] (fp16 bit patterns).  s1 and z [N, K/128] receive
 * the canonical group parameters when non-NULL (for inspection and tests).
 * w, wpacked and s0_fp16 are required. */
w4a8_status quantize_weights_w4g128(const float *w, int64_t N, int64_t K,
                                    void *wpacked, uint8_t *s1, uint8_t *z,
                                    uint16_t *s0_fp16, hipStream_t stream);

/* Inverse of the packing step: rebuild the canonical codes from a device
 * weight stream.  q4_canon [N, K/2]: byte (n, k/2) holds q4[n,k] for even k
 * in its low nibble and q4[n,k+1] in its high nibble.  s1, z [N, K/128].
 * All pointers required.  For tests and inspection. */
w4a8_status w4a8_unpack_weights(const void *wpacked, int64_t N, int64_t K,
                                uint8_t *q4_canon, uint8_t *s1, uint8_t *z,
                                hipStream_t stream);

/* ------------------------------------------------------------------------
 * Per-token INT8 activation quantization (QServe talk summary, "Precision
 * Data Flow and Activation Quantization Fusion": every linear layer takes
 * 8-bit activations).
 *   s_a[m] = max_k |x[m,k]| / 127   (fp32 division)
 *   qx[m,k] = clamp(rint(x[m,k] / s_a[m]), -127, 127)   (0 if s_a == 0)
 * x_fp16: [M, K] fp16 bit patterns, row stride ldx >= K elements (ldx must
 * be a multiple of 8).  qx: [M, K] int8, row stride K.  s_a: [M] fp32.
 * ------------------------------------------------------------------------ */
w4a8_status quantize_act_per_token_i8(const uint16_t *x_fp16, int64_t M,
                                      int64_t K, int64_t ldx, int8_t *qx,
                                      float *s_a, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Normalization fused with the per-token INT8 quantization (QServe talk
 * summary, "Precision Data Flow and Activation Quantization Fusion": the
 * quantization is folded into the preceding layer, e.g. LayerNorm, which
 * then writes the 8-bit activations directly).  Per token m:
 *   LayerNorm (rms == 0): mean = exact row sum (in units of 2^-24) * 2^-24 / K
 *                         (double); RMSNorm (rms == 1): mean = 0
 *   var  = sum_k (double(x[m,k]) - mean)^2 / K          (double)
 *   rstd = float(1 / sqrt(var + eps))   (0 when var + eps == 0)
 *   h[k] = fp16_rne(((float(x) - float(mean)) * rstd) * float(gamma[k])
 *                   + float(beta[k]))    (fp32, in that order; no beta: no add)
 * then qx[m,:] and s_a[m] from h exactly as quantize_act_per_token_i8 would
 * compute them from an fp16 row h.  The second moment is summed in double in
 * a tree over lanes, so rstd may differ from a sequential sum's only when the
 * double 1/sqrt lies within about K * 2^-53 (relative) of a midpoint between
 * two floats.
 * x_fp16: [M, K] fp16 bit patterns, row stride ldx >= K (multiple of 8).
 * gamma_fp16: [K] fp16, required.  beta_fp16: [K] fp16 or NULL (no shift).
 * eps: finite, >= 0.  rms: 0 or 1.  qx: [M, K] int8, row stride K; s_a: [M]
 * fp32.  K <= 2^20 (W4A8_E_SHAPE otherwise) keeps the exact row sum in 64
 * bits.  The normalized values must be finite in fp16 (larger results are
 * unspecified, as for non-finite inputs).
 * ------------------------------------------------------------------------ */
w4a8_status norm_quantize_act_i8(const uint16_t *x_fp16, int64_t M, int64_t K,
                                 int64_t ldx, const uint16_t *gamma_fp16,
                                 const uint16_t *beta_fp16, float eps, int rms,
                                 int8_t *qx, float *s_a, hipStream_t stream);

/* ------------------------------------------------------------------------
 * W4A8 GEMM (QServe talk summary, "Quantized Matrix Multiplication (GEMM)
 * Kernel on GPUs" and "Challenges and Design Details of QServe GEMM Kernel";
 * Lecture 15 notes, 15.5-15.6).
 *   acc[m,n] = sum_k qx[m,k] * (q4[n,k]*s1[n,k/128] - z[n,k/128]*s1[n,k/128])
 *              (exact, INT32)
 *   y[m,n]   = fp16_rne((float(acc) * s_a[m]) * float(s0[n]))
 * qx [M, K] int8 and s_a [M] fp32 as written by quantize_act_per_token_i8;
 * wpacked and s0_fp16 as written by quantize_weights_w4g128.
 * y_fp16: [M, N] fp16 bit patterns, row-major.  acc_out: optional [M, N]
 * int32, row-major; when non-NULL the raw accumulators of the same main loop
 * are written too.
 * ws: workspace of at least gemm_w4a8_workspace_bytes(M, N, K) bytes, zeroed
 * by the caller once after allocation; every call leaves its counters zeroed
 * again.  It holds the split-K partial sums of decode shapes and the
 * stream-K counters and partial tiles of prefill shapes.  ws may be NULL:
 * the call then runs a plan that does not split K (the default plan unsplit
 * when its LDS still fits, else the best-scored unsplit plan; same results,
 * slower for shapes whose tiles do not fill the GPU; gemm_w4a8_plan_detail
 * with with_workspace = 0 names it).  A non-NULL ws smaller than required is
 * W4A8_E_WORKSPACE.  Calls that share one workspace must be ordered (same
 * stream, or synchronised): concurrent calls on one workspace race.
 * ------------------------------------------------------------------------ */
size_t gemm_w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K);

w4a8_status gemm_w4a8(const int8_t *qx, const float *s_a, const void *wpacked,
                      const uint16_t *s0_fp16, int64_t M, int64_t N, int64_t K,
                      uint16_t *y_fp16, int32_t *acc_out, void *ws,
                      size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * gemm_w4a8 for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The same plan,
 * kernels and results as gemm_w4a8 with a workspace, but the split-K /
 * stream-K workspace is a fixed array in device memory inside the library
 * (W4A8_NOALLOC_SCRATCH_BYTES on every device the library runs on, held
 * until the process ends).  The call allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine.  Its first call on a device looks
 * up that device's copy of the array and clears its counters with a small
 * kernel on `stream`.
 * Every call on one device shares that device's array: calls that overlap
 * on one GPU (different streams, or concurrent host threads without ordering)
 * race and may give wrong results; order them on one stream.  The array is
 * left as the last call used it (its counters zero).
 * A shape whose plan needs more workspace than the array holds (see
 * gemm_w4a8_workspace_bytes) is rejected with W4A8_E_SCRATCH before any
 * launch.  Other arguments as gemm_w4a8; the stream must belong to the
 * current device.
 * ------------------------------------------------------------------------ */
#define W4A8_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

w4a8_status gemm_w4a8_noalloc(const int8_t *qx, const float *s_a, const void *wpacked,
                              const uint16_t *s0_fp16, int64_t M, int64_t N, int64_t K,
                              uint16_t *y_fp16, int32_t *acc_out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Measurement aid: the streaming-read ceiling (Lecture 15 notes, 15.1 and
 * "Numbers worth memorizing": a decode-size layer cannot finish before its
 * weight bytes have streamed from HBM).  Reads `bytes` of device memory at
 * `buf` once, the way the GEMM reads its weight stream (16-byte
 * non-temporal loads, 32 KB per workgroup, every load of a wave in flight at
 * once), and computes nothing from them; its duration on the same number of
 * bytes is the fastest a streaming kernel launch reaches on the device, the
 * second yardstick (beside the published HBM peak) for the decode GEMM.
 * bytes % 16 == 0 and bytes < 2^31 (W4A8_E_SHAPE otherwise; 0 is a no-op);
 * buf 16-byte aligned, sink one 4-byte-aligned device dword that is written
 * only in the (practically never taken) case that the data's xor equals a
 * fixed constant.
 * ------------------------------------------------------------------------ */
w4a8_status w4a8_hbm_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Plan introspection and the learned plan selector (host only; no GPU work).
 *
 * gemm_w4a8_plan: the plan gemm_w4a8 would launch for (M, N, K) on the
 * current device: desc[0..7] = kind (0 streamed-weight decode kernel, 1
 * matrix-core kernel), m-tiles (TM for kind 1), n-tiles, split-K (stream-K
 * ranges for kind 1), waves, pipeline depth, staged activations (0/1),
 * workspace bytes, waves splitting N instead of K (0/1).
 *
 * gemm_w4a8_plan_detail: the same for a call with a workspace
 * (with_workspace = 1) or with ws == NULL (with_workspace = 0), plus
 * desc[9] = the dynamic LDS bytes per workgroup its launch requests.
 *
 * gemm_w4a8_decode_candidates: the decode-kernel plans that can run (M <=
 * 1024; gemm_w4a8 takes the decode kernels up to 64 tokens, up to 128 when
 * the prefill kernel's 64 x 256 tiles would fill under half of the compute
 * units, and up to 1024 when M x N is at most 2^20 as well, except on very
 * large weights whose four-m-tile workgroups would take two rounds, or at
 * most 2^21 with N x K at most 2^25; past 256 tokens only N x K up to 2^25,
 * past 512 up to 2^23): *count
 * is their number; the first max_plans are written to plans as rows of
 * seven int32 (m-tiles, n-tiles, split-K, waves, depth, staged, waves
 * splitting N).  Each row, set in W4A8_DECODE_PLAN as
 * "mt,nt,splitk,waves,depth,staged,wave_n", makes gemm_w4a8 run that plan
 * on the decode kernels at any M <= 1024 (for tuning sweeps).
 *
 * gemm_w4a8_selector_score: the compiled-in model's predicted fraction of the
 * HBM peak for one such plan row on a device with `cus` compute units, or a
 * negative value when no model is compiled in or the arguments are invalid.
 * The model follows the QFactory reading notes (6.2, "ML-based kernel
 * selector"): a small multilayer perceptron over the matrix shape and the
 * tiling parameters, trained on measured bandwidth utilization; gemm_w4a8
 * takes the candidate it scores highest at 1..64 tokens (W4A8_SELECTOR=0
 * restores the fixed rules; past 64 tokens fixed decision trees pick).
 * ------------------------------------------------------------------------ */
w4a8_status gemm_w4a8_plan(int64_t M, int64_t N, int64_t K, int64_t *desc);   /* desc: 9 int64 */

w4a8_status gemm_w4a8_plan_detail(int64_t M, int64_t N, int64_t K, int with_workspace,
                                  int64_t *desc);   /* desc: 10 int64 */

w4a8_status gemm_w4a8_decode_candidates(int64_t M, int64_t N, int64_t K, int32_t *plans,
                                        int32_t max_plans, int32_t *count);

float gemm_w4a8_selector_score(int64_t M, int64_t N, int64_t K, const int32_t *plan, int64_t cus);

/* ------------------------------------------------------------------------
 * W4A16 GEMM on the same weights: fp16 activations, no activation
 * quantization; the weights are dequantized to fp16 inside the main loop
 * (QFactory reading notes, 2.1: w = (w_quant - zero) * scale; Lecture 15
 * notes, 15.5: the int4 -> fp16 path).  With the two-level weights the
 * dequantized weight is r * s0[n], r = q4*s1 - z*s1 (an integer in
 * [-127, 127]):
 *   y[m,n] = fp16_rne( float(s0[n]) * sum_k x[m,k] * r[n,k] )
 * with every product exact and the sum accumulated in fp32 on the matrix
 * cores (order unspecified, deterministic run to run).
 * x_fp16: [M, K] fp16, row stride ldx >= K (a multiple of 8).  wpacked and
 * s0_fp16 as written by quantize_weights_w4g128.  y_fp16: [M, N] fp16,
 * row-major.  Built for few tokens (the weight stream is read once per 16
 * tokens).
 * ------------------------------------------------------------------------ */
w4a8_status gemm_w4a16(const uint16_t *x_fp16, int64_t M, int64_t K, int64_t ldx,
                       const void *wpacked, const uint16_t *s0_fp16, int64_t N,
                       uint16_t *y_fp16, hipStream_t stream);

/* ------------------------------------------------------------------------
 * 4-bit KV cache and decode attention over it.
 *
 * Format (QServe talk summary, "Smooth Attention for K4V4 KV Cache
 * Compression", "Attention Computation Acceleration", "Long Context
 * Challenges": 4-bit keys and values with per-token zero points and scales;
 * QFactory reading notes, 2.1: x ~ (code - zero) * scale).  Every (token,
 * kv head) row of head_dim = 128 values is quantized on its own:
 *   lo = min(0, min x), hi = max(0, max x)
 *   scale = fp16_rne((hi - lo) / 15)            (fp32 subtraction, IEEE division)
 *   zero  = clamp(rint(-lo / scale), 0, 15)     (fp32, ties to even)
 *   code  = clamp(rint(x / scale) + zero, 0, 15)
 * and a row whose scale rounds to 0 stores scale 0, zero 0 and codes 0.
 * Inputs must be finite.
 *
 * A cache is one device buffer of kv4_cache_bytes(B, Hkv, S) bytes for the
 * keys and one of the same size for the values, for B sequences, Hkv kv heads
 * and a capacity of S tokens (S > 0, a multiple of 32).  Its layout is
 * private (read it back with kv4_unpack); only its size is part of the ABI.
 * Caches are caller-owned device memory; their content before the first
 * write is irrelevant.
 * ------------------------------------------------------------------------ */
size_t kv4_cache_bytes(int64_t B, int64_t Hkv, int64_t S);

/* Quantize T new tokens per sequence and write them into the caches at
 * positions pos[b] .. pos[b] + T - 1 (pos: device int32 [B]; tokens at or
 * past the capacity S, and sequences with pos[b] < 0, are not written).
 * k_fp16, v_fp16: [B, T, Hkv, 128] fp16, contiguous (the layout of a fused
 * QKV projection's K and V columns for T tokens of each sequence).  Calls
 * that write the same cache must be ordered on one stream. */
w4a8_status quantize_kv4(const uint16_t *k_fp16, const uint16_t *v_fp16, int64_t B, int64_t Hkv,
                         int64_t T, const int32_t *pos, void *k_cache, void *v_cache, int64_t S,
                         hipStream_t stream);

/* Test inverse of the cache layout: the logical codes [B, Hkv, S, 128] (one
 * per byte), scales [B, Hkv, S] (fp16 bits) and zeros [B, Hkv, S] of one
 * cache (is_v = 0: a key cache, 1: a value cache). */
w4a8_status kv4_unpack(const void *cache, int is_v, int64_t B, int64_t Hkv, int64_t S,
                       uint8_t *codes, uint16_t *scales_fp16, uint8_t *zeros, hipStream_t stream);

/* Decode attention: one query token per sequence over the first lens[b]
 * cached tokens (lens: device int32 [B]; values above S are taken as S,
 * negative ones as 0).  For query head h, kv head g = h / (Hq / Hkv)
 * (consecutive query heads share a kv head; Hq / Hkv <= 16):
 *   score_t = sm_scale * sum_d q[d] * (kcode[t,d] - kzero[t]) * kscale[t]
 *   out[d]  = sum_t softmax(score)_t * (vcode[t,d] - vzero[t]) * vscale[t]
 * and out = 0 when lens[b] = 0.  q_fp16: [B, Hq, 128] fp16; out_fp16:
 * [B, Hq, 128] fp16.  Scores accumulate exact products in fp32; the
 * softmax runs in fp32 base 2 over chunks of 256 tokens; the value sum takes
 * fp16(p_t * vscale[t] * 2^E) (2^E a per-chunk power of two) against the
 * exact (code - zero).  The error bound that follows is stated with the
 * tests.  ws: kv4_attention_workspace_bytes(B, Hq, S) bytes of device memory
 * (chunk partial sums; scratch, no initial content) or NULL when that is 0;
 * a smaller size is W4A8_E_WORKSPACE.  Calls sharing ws must be ordered. */
size_t kv4_attention_workspace_bytes(int64_t B, int64_t Hq, int64_t S);

w4a8_status attention_kv4_decode(const uint16_t *q_fp16, int64_t B, int64_t Hq, int64_t Hkv,
                                 const void *k_cache, const void *v_cache, int64_t S,
                                 const int32_t *lens, float sm_scale, uint16_t *out_fp16,
                                 void *ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A8_H */
