/*
 * qgemv — block-quantized decode GEMV for AMD Instinct MI355X (gfx950).
 *
 * Single-token (and up to 4-token) autoregressive decode turns each
 * projection into a matrix-vector product over weights that stay in their
 * quantized form in HBM and are widened only in registers, next to the
 * multiply.  Sources for the operation:
 *   - "Decode 只有一行" (decode has only one row) and the "W8 直读"
 *     (W8 direct read) section of the zLLM GLM-5.3 ROCm decode post on
 *     juejin: decode is a GEMV bound by weight bandwidth, and the kernel
 *     should consume W8 codes plus scales directly rather than a widened
 *     copy; the post's bottleneck table names contiguous wide reads of the
 *     weight stream as the lever.
 *   - "Qwen3-14B TP4 W8A16 Decode" in the Qwen3 C++ Reference Runtime
 *     (MetaInfer-cpp) README: signed int8 weights, bf16 activations, fp32
 *     accumulation; "Decode small-M Linear": M = 1..4 activation rows share
 *     one pass over the weights, with a strided input row.
 *   - The W4A16 reading in the commit log of vllm.cpp pull request #1936
 *     ("perf(GFX1100-TG200)"): activations stay bf16 and the weights are
 *     dequantized inside the GEMV's registers.
 *
 * Formats (canonical, row-major, one output row n per weight row):
 *   Q8G64:  q[N][K] int8; scale[N][K/64] fp16 bit patterns;
 *           w[n][k] = q[n][k] * scale[n][k/64]
 *   Q8G128: as Q8G64 with one scale per 128 K (scale[N][K/128]); the
 *           LM-head format of the zLLM post's per-operator format map
 *   Q8PC:   q[N][K] int8, one fp32 scale per output row (scale[N]);
 *           w[n][k] = q[n][k] * scale[n]; the per-output-channel W8A16
 *           format of the MetaInfer-cpp README (K a multiple of 16 here)
 *   Q4G32:  codes[N][K/2] bytes, element k in the low nibble of byte k/2 when
 *           k is even, the high nibble when k is odd; scale[N][K/32] and
 *           min[N][K/32] fp16 bit patterns; w[n][k] = code * scale + min
 * The GEMV computes, for activation rows i < m,
 *          y[i*ldy + n] = sum_k w[n][k] * x[i*ldx + k]
 * with x in bf16 bit patterns and y in fp32.  Accumulation is fp32 in an
 * unspecified but fixed order: a result is bit-identical from run to run.
 *
 * Ownership: the caller owns every buffer.  The library never allocates,
 * frees or synchronizes.  qpack_* and qunpack_* work on host memory only;
 * qgemv_* take device pointers, validate everything they can on the host,
 * enqueue one kernel on the given HIP stream (NULL = the default stream) and
 * return without waiting.  On any error nothing is enqueued.  No C++
 * exception crosses this interface.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Version of this interface and of the packed layouts: a buffer packed by
 * qpack_* is valid input only for a library of the same version.  Version 2
 * stores 8-bit codes unbiased (signed, as given). */
#define QG_ABI_VERSION 2

/* Result of every call that can fail.  Errors are returned, never thrown and
 * never answered by running some other path: the explicit Status / Result
 * propagation of the MetaInfer-cpp (Qwen3 C++ Reference Runtime) README,
 * milestone "M1 Core 与 Backend", whose HIP backend returns Unsupported
 * instead of falling back to the CPU.  Validation (shape, stride, alignment,
 * byte range) happens on the host before anything is enqueued, after that
 * section's validated TensorView. */
typedef enum qg_status {
    QG_OK = 0,
    QG_ERR_INVALID_ARG = 1,  /* null pointer, bad size, stride or buffer length */
    QG_ERR_UNSUPPORTED = 2,  /* valid request outside what is built (m > 4, ...) */
    QG_ERR_ALIGNMENT = 3,    /* a pointer or stride breaks an alignment rule */
    QG_ERR_HIP = 4,          /* the HIP runtime reported an error at launch */
    /* Reserved, never returned: they make every int a valid qg_status value
     * (C++ leaves an enum holding a value outside its range undefined, and
     * a status read from elsewhere may hold anything). */
    QG_STATUS_RESERVED_MIN_ = -2147483647 - 1,
    QG_STATUS_RESERVED_MAX_ = 2147483647
} qg_status;

/* Human-readable name of a status code (the same "M1 Core 与 Backend"
 * convention); "unknown status" for a value outside the enum; never NULL. */
const char *qg_status_string(qg_status status);

/* QG_ABI_VERSION of the built library. */
int qg_abi_version(void);

/* ------------------------------------------------------------------ packing
 * qpack_* re-tile canonical weights, once per matrix, into the layout the
 * kernels stream with 16-byte loads per lane.  The layout is fixed once, at
 * load time (the WeightArchive of the MetaInfer-cpp README, milestone "M2
 * Model Inputs 与 Weight Loading", materialises weights once in 256-byte
 * aligned storage), and only whole rows move (the commit log of vllm.cpp
 * pull request #1936 notes that row permutation is safe for block formats,
 * while column permutation crosses groups).  Row order and the grouping
 * along K are kept; the packed buffer is opaque and its size depends only
 * on (N, K).  K must be a whole number of groups (64 for Q8G64, 128 for
 * Q8G128, 32 for Q4G32, 16 for Q8PC) and 1 <= N, K < 2^31.
 *
 * *_size returns the packed size in bytes (a multiple of 256), or 0 for an
 * invalid shape.  The device copy of a packed buffer must be 256-byte
 * aligned.  qpack_* return QG_ERR_INVALID_ARG for a null pointer, an invalid
 * shape or out_bytes < *_size(N, K); they write exactly *_size bytes.
 * qunpack_* invert qpack_* byte for byte (for inspection and tests). */
size_t    qpack_q8g64_size(int64_t N, int64_t K);
qg_status qpack_q8g64(const int8_t *q, const uint16_t *scales_f16,
                      int64_t N, int64_t K, void *out, size_t out_bytes);
qg_status qunpack_q8g64(const void *packed, size_t packed_bytes, int64_t N, int64_t K,
                        int8_t *q, uint16_t *scales_f16);

size_t    qpack_q8g128_size(int64_t N, int64_t K);              /* K % 128 == 0 */
qg_status qpack_q8g128(const int8_t *q, const uint16_t *scales_f16,
                       int64_t N, int64_t K, void *out, size_t out_bytes);
qg_status qunpack_q8g128(const void *packed, size_t packed_bytes, int64_t N, int64_t K,
                         int8_t *q, uint16_t *scales_f16);

size_t    qpack_q8pc_size(int64_t N, int64_t K);                /* K % 16 == 0 */
qg_status qpack_q8pc(const int8_t *q, const float *scales_f32,
                     int64_t N, int64_t K, void *out, size_t out_bytes);
qg_status qunpack_q8pc(const void *packed, size_t packed_bytes, int64_t N, int64_t K,
                       int8_t *q, float *scales_f32);

size_t    qpack_q4g32_size(int64_t N, int64_t K);
qg_status qpack_q4g32(const uint8_t *codes, const uint16_t *scales_f16,
                      const uint16_t *mins_f16, int64_t N, int64_t K,
                      void *out, size_t out_bytes);
qg_status qunpack_q4g32(const void *packed, size_t packed_bytes, int64_t N, int64_t K,
                        uint8_t *codes, uint16_t *scales_f16, uint16_t *mins_f16);

/* Gate/up pair packing for qgemv_grouped_q4g32_swiglu: the gate and up
 * projections of one expert (each N x K, Q4G32, canonical as above) in one
 * buffer whose tiles hold matching gate and up rows side by side, so the
 * kernel that ends a tile holds both halves of each output.  This is the
 * row-stacked gate+up matrix of the merged gate_up GEMM in the commit log of
 * vllm.cpp pull request #1936 (rows are independent, so stacking them keeps
 * every row's result), interleaved in blocks of rows instead of appended.
 * Size rules as qpack_q4g32 (K % 32 == 0). */
size_t    qpack_q4g32_gate_up_size(int64_t N, int64_t K);
qg_status qpack_q4g32_gate_up(const uint8_t *gate_codes, const uint16_t *gate_scales_f16,
                              const uint16_t *gate_mins_f16, const uint8_t *up_codes,
                              const uint16_t *up_scales_f16, const uint16_t *up_mins_f16,
                              int64_t N, int64_t K, void *out, size_t out_bytes);
qg_status qunpack_q4g32_gate_up(const void *packed, size_t packed_bytes, int64_t N, int64_t K,
                                uint8_t *gate_codes, uint16_t *gate_scales_f16,
                                uint16_t *gate_mins_f16, uint8_t *up_codes,
                                uint16_t *up_scales_f16, uint16_t *up_mins_f16);

/* ------------------------------------------------------------------- GEMV
 * y[i*ldy + n] = sum_k W[n][k] * x[i*ldx + k] for 0 <= i < m, 0 <= n < N.
 *   w_packed  device, qpack_*_size(N, K) bytes from qpack_*, 256-B aligned
 *   x_bf16    device, m rows of K bf16 values, row stride ldx elements;
 *             4-byte aligned, ldx even when m > 1
 *   y         device fp32, m rows of N values, row stride ldy elements;
 *             4-byte aligned; only y[i*ldy + n] for n < N is written
 *   m         1..4 (QG_ERR_UNSUPPORTED otherwise)
 *   ldx >= K, ldy >= N
 *   hip_stream  a hipStream_t, or NULL for the default stream
 * K * m is further limited by the 160 KB of LDS a work-group may hold
 * (activations plus per-unit activation sums); larger requests return
 * QG_ERR_UNSUPPORTED. */
qg_status qgemv_q8g64(const void *w_packed, const uint16_t *x_bf16, float *y,
                      int64_t m, int64_t N, int64_t K, int64_t ldx, int64_t ldy,
                      void *hip_stream);
qg_status qgemv_q4g32(const void *w_packed, const uint16_t *x_bf16, float *y,
                      int64_t m, int64_t N, int64_t K, int64_t ldx, int64_t ldy,
                      void *hip_stream);
/* Same contract for the two further 8-bit formats (packed by qpack_q8g128 /
 * qpack_q8pc with the same N and K). */
qg_status qgemv_q8g128(const void *w_packed, const uint16_t *x_bf16, float *y,
                       int64_t m, int64_t N, int64_t K, int64_t ldx, int64_t ldy,
                       void *hip_stream);
qg_status qgemv_q8pc(const void *w_packed, const uint16_t *x_bf16, float *y,
                     int64_t m, int64_t N, int64_t K, int64_t ldx, int64_t ldy,
                     void *hip_stream);

/* ------------------------------------------------- batched decode, m <= 16
 * Decode with up to 16 activation rows on the matrix cores: the larger-batch
 * ("B8/B16") decode of the Qwen3 C++ Reference Runtime (MetaInfer-cpp)
 * README, where the input rows are reused from LDS across every weight.  The
 * weights use their own packed layout (one 1 KiB wave load = 16 rows x 64 K,
 * the MFMA operand order), made by qpack_*_mma; y is the same product as the
 * plain GEMV:
 *   y[i*ldy + n] = sum_k W[n][k] * x[i*ldx + k],  0 <= i < m, 2 <= m <= 16.
 * K must be a multiple of 64 (128 for Q8G128).  The m activation rows are
 * staged in LDS when they fit (m * K * 2 bytes, plus K * 2 for Q4G32's
 * per-group activation sums, within 159 KiB, less the partial sums of a K
 * split); longer rows are read from memory with each
 * weight item instead, so any K is accepted.  Pointers, strides, ownership
 * and errors as qgemv_q8g64, with m = 2..16: m = 1 returns
 * QG_ERR_UNSUPPORTED (single-token decode has no matrix to feed the matrix
 * cores and takes the qgemv_* calls above; m = 0 does nothing).  Each output
 * row is computed on its own (rows do not affect one another's bits). */
size_t    qpack_q8g64_mma_size(int64_t N, int64_t K);
size_t    qpack_q8g128_mma_size(int64_t N, int64_t K);
size_t    qpack_q8pc_mma_size(int64_t N, int64_t K);
qg_status qpack_q8g64_mma(const int8_t *q, const uint16_t *scales_f16, int64_t N, int64_t K,
                          void *out, size_t out_bytes);
qg_status qpack_q8g128_mma(const int8_t *q, const uint16_t *scales_f16, int64_t N, int64_t K,
                           void *out, size_t out_bytes);
qg_status qpack_q8pc_mma(const int8_t *q, const float *scales_f32, int64_t N, int64_t K,
                         void *out, size_t out_bytes);
qg_status qunpack_q8g64_mma(const void *packed, size_t packed_bytes, int64_t N, int64_t K,
                            int8_t *q, uint16_t *scales_f16);
qg_status qunpack_q8g128_mma(const void *packed, size_t packed_bytes, int64_t N, int64_t K,
                             int8_t *q, uint16_t *scales_f16);
qg_status qunpack_q8pc_mma(const void *packed, size_t packed_bytes, int64_t N, int64_t K,
                           int8_t *q, float *scales_f32);
qg_status qgemv_q8g64_mma(const void *w_packed, const uint16_t *x_bf16, float *y, int64_t m,
                          int64_t N, int64_t K, int64_t ldx, int64_t ldy, void *hip_stream);
qg_status qgemv_q8g128_mma(const void *w_packed, const uint16_t *x_bf16, float *y, int64_t m,
                           int64_t N, int64_t K, int64_t ldx, int64_t ldy, void *hip_stream);
qg_status qgemv_q8pc_mma(const void *w_packed, const uint16_t *x_bf16, float *y, int64_t m,
                         int64_t N, int64_t K, int64_t ldx, int64_t ldy, void *hip_stream);
/* Q4G32 on the matrix cores, same contract: one MFMA per 32-group, whose
 * B operand is the group's codes less the group's zero point
 * z = clamp(rint(-min / scale), 0, 15), widened to bf16 exactly; that sum is
 * scaled and (min + scale * z) times the group's activation sum is added,
 * so neither term can cancel (each is at most twice the largest weight of
 * the group in size).  Packed by qpack_q4g32_mma
 * (1 KiB wave load = 16 rows x 128 K); K must be a multiple of 128 (else
 * QG_ERR_INVALID_ARG).  codes, scales and mins are the canonical Q4G32
 * arrays of qpack_q4g32. */
size_t    qpack_q4g32_mma_size(int64_t N, int64_t K);
qg_status qpack_q4g32_mma(const uint8_t *codes, const uint16_t *scales_f16,
                          const uint16_t *mins_f16, int64_t N, int64_t K, void *out,
                          size_t out_bytes);
qg_status qunpack_q4g32_mma(const void *packed, size_t packed_bytes, int64_t N, int64_t K,
                            uint8_t *codes, uint16_t *scales_f16, uint16_t *mins_f16);
qg_status qgemv_q4g32_mma(const void *w_packed, const uint16_t *x_bf16, float *y, int64_t m,
                          int64_t N, int64_t K, int64_t ldx, int64_t ldy, void *hip_stream);

/* Routed-expert decode (one token, several experts), Q4G32:
 *   for each slot j < n_slots, with e = expert_ids_dev[j]:
 *     y[j*y_slot_stride + n] = sum_k W_e[n][k] * x[j*x_slot_stride + k]
 *   Each slot's output is written separately; nothing is combined across
 *   slots.  The sources motivate this as the routed-expert weight streams of
 *   the zLLM post's bottleneck table and per-operator format map.
 *   w_experts_packed  device, n_experts packed matrices (each from
 *                     qpack_q4g32 with this N, K), matrix e at byte offset
 *                     e * expert_stride_bytes; 256-B aligned
 *   expert_stride_bytes  multiple of 256, >= qpack_q4g32_size(N, K)
 *   expert_ids_dev    device int32[n_slots]; read by the kernel, not the
 *                     host.  A slot whose id is outside [0, n_experts)
 *                     streams no weights (it may read the first work item
 *                     of matrix 0, never memory outside the buffer) and
 *                     has its N outputs set to NaN.
 *   n_slots           1..64
 *   x_slot_stride     elements between slot activations; 0 = one shared x
 *                     (gate and up projections); even
 *   y_slot_stride     elements between slot outputs, >= N
 * Same alignment and LDS rules as qgemv_q4g32 with m = 1. */
qg_status qgemv_grouped_q4g32(const void *w_experts_packed, int64_t expert_stride_bytes,
                              int32_t n_experts, const int32_t *expert_ids_dev,
                              int32_t n_slots, const uint16_t *x_bf16, int64_t x_slot_stride,
                              float *y, int64_t y_slot_stride, int64_t N, int64_t K,
                              void *hip_stream);

/* Routed-expert gate+up projection with the SwiGLU activation fused into
 * its epilogue (one token, several experts), Q4G32:
 *   for each slot j < n_slots, with e = expert_ids_dev[j] and x_j the slot's
 *   activation,
 *     g = Gate_e x_j,  u = Up_e x_j  (fp32, computed as qgemv_grouped_q4g32)
 *     act[j*act_slot_stride + n] = bf16( silu(g[n]) * u[n] ),
 *     silu(z) = z / (1 + exp(-z)),  rounded to nearest even
 *   for 0 <= n < N.  act is laid out as the activation input of the down
 *   projection's grouped call (x_slot_stride = act_slot_stride).  The
 *   "packed Gate/Up GEMM, then one kernel computes SwiGLU and writes the
 *   down projection's input" step is from the Qwen3 C++ Reference Runtime
 *   (MetaInfer-cpp) README, milestone M6.5-D; here the GEMV and the
 *   activation are one kernel and g, u never reach memory.
 *   w_gate_up_packed  device, n_experts buffers from qpack_q4g32_gate_up
 *                     (this N, K), buffer e at byte offset
 *                     e * expert_stride_bytes; 256-B aligned
 *   expert_stride_bytes  multiple of 256, >= qpack_q4g32_gate_up_size(N, K)
 *   expert_ids_dev    as qgemv_grouped_q4g32; a slot with an id outside
 *                     [0, n_experts) streams no weights (as there) and
 *                     gets NaN (0x7FC0)
 *   act_bf16          device bf16, 2-byte aligned; act_slot_stride >= N
 *   n_slots, x_bf16, x_slot_stride, K: as qgemv_grouped_q4g32. */
qg_status qgemv_grouped_q4g32_swiglu(const void *w_gate_up_packed, int64_t expert_stride_bytes,
                                     int32_t n_experts, const int32_t *expert_ids_dev,
                                     int32_t n_slots, const uint16_t *x_bf16,
                                     int64_t x_slot_stride, uint16_t *act_bf16,
                                     int64_t act_slot_stride, int64_t N, int64_t K,
                                     void *hip_stream);

/* ------------------------------------------------------------ greedy tail
 * Greedy token choice over fp32 logits (the LM head's output):
 *   idx_out[i] = the n in [0, N) with the largest x[i*ldx + n], the lowest
 *                such n on ties, for 0 <= i < m.
 * Values compare as real numbers (-0 == +0; -inf lowest); a NaN counts as
 * larger than every number, so the first NaN of a row wins.  Each row is
 * split across work-groups with a (value, lower index) comparator, the
 * split argmax of the commit log of vllm.cpp pull request #1936 (also the
 * device-side greedy step after the LM head in the Qwen3 C++ Reference
 * Runtime (MetaInfer-cpp) README, milestone M6.5-F); the index does not
 * depend on the split or on timing.  One kernel launch.
 *   x          device fp32, 4-byte aligned, m rows of N values, ldx >= N
 *   idx_out    device int32[m], 4-byte aligned
 *   workspace  device, >= qg_argmax_workspace_size(m) bytes, 8-byte
 *              aligned, all zero before the first call.  Each completed
 *              call leaves it all zero again.  Calls that share a workspace
 *              must not overlap in time (same stream is enough).
 *   1 <= N < 2^31; m = 0 is a no-op; m <= 65535. */
size_t    qg_argmax_workspace_size(int64_t m);
qg_status qg_argmax_f32(const float *x, int64_t m, int64_t N, int64_t ldx, int32_t *idx_out,
                        void *workspace, size_t workspace_bytes, void *hip_stream);

/* LM head with the greedy choice fused into the GEMV: as qgemv_q8g64 /
 * qgemv_q8g128, and in the same launch idx_out[i] = the argmax of output
 * row i under the rule of qg_argmax_f32.  The fused LM-head argmax candidate
 * of the Qwen3 C++ Reference Runtime (MetaInfer-cpp) README, milestone
 * M6.5-F (rejected there against a library GEMM plus argmax; here the GEMV
 * is this library's own).  The index equals qg_argmax_f32 applied to the
 * logits the same call writes.
 *   logits     device fp32 m x N with row stride ldy, or NULL to skip
 *              writing the logits (ldy is then ignored)
 *   idx_out    device int32[m]
 *   workspace  as qg_argmax_f32 (qg_argmax_workspace_size(m) bytes, zero
 *              before the first call, left zero by every completed call;
 *              calls sharing it must not overlap)
 * Other arguments and errors as qgemv_q8g64. */
qg_status qgemv_q8g64_argmax(const void *w_packed, const uint16_t *x_bf16, float *logits,
                             int32_t *idx_out, int64_t m, int64_t N, int64_t K, int64_t ldx,
                             int64_t ldy, void *workspace, size_t workspace_bytes,
                             void *hip_stream);
qg_status qgemv_q8g128_argmax(const void *w_packed, const uint16_t *x_bf16, float *logits,
                              int32_t *idx_out, int64_t m, int64_t N, int64_t K, int64_t ldx,
                              int64_t ldy, void *workspace, size_t workspace_bytes,
                              void *hip_stream);

/* Allocation-free LM head with the fused greedy choice, for callers that
 * cannot allocate or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): qgemv_q8g64_argmax
 * without the workspace arguments.  The keys and counter live in a small
 * device array owned by the library (256 bytes per GPU, held until the
 * process ends); the first call on a device looks up that GPU's copy and
 * enqueues one small kernel that zeroes it, and every completed call leaves
 * it zeroed again.  Nothing is allocated or freed.  Calls that overlap in
 * time on one GPU share the array and race: issue them on one stream (or
 * otherwise serialize them).  m = 1..4 (the array holds the workspace of at
 * most 4 rows; QG_ERR_UNSUPPORTED beyond); other arguments, results and
 * errors as qgemv_q8g64_argmax; QG_ERR_HIP if the array cannot be found. */
qg_status qgemv_q8g64_argmax_noalloc(const void *w_packed, const uint16_t *x_bf16, float *logits,
                                     int32_t *idx_out, int64_t m, int64_t N, int64_t K, int64_t ldx,
                                     int64_t ldy, void *hip_stream);

/* ------------------------------------------------------------- test hooks
 * Host-side route counters, after the routing witnesses of the vllm.cpp pull
 * request #1936 commit log (process-global counters bumped once per dispatch
 * on exactly the branch taken, with a reset hook, so that tests can assert
 * which kernel ran).  Every successful qgemv_* call bumps the counter of the
 * kernel variant it launched.  Variant names: "<fmt>[_grouped[_swiglu]|_argmax]_m<m>_g<G>_r<R>"
 * with fmt one of q8g64, q4g32, q8g128, q8pc, e.g. "q8g64_m1_g32_r2".
 * qg_route_count returns 0 for unknown names. */
void     qg_route_counts_reset(void);
uint64_t qg_route_count(const char *variant);
/* Writes the name of the variant qgemv_* would launch for (fmt, m, N, K)
 * (one distinct kernel symbol per variant, so that a profile never averages
 * two of them under one name: the symbol-collision lesson of the vllm.cpp
 * pull request #1936 commit log)
 * into buf (fmt 0 = Q8G64, 1 = Q4G32, 2 = grouped Q4G32, 3 = Q8G128,
 * 4 = Q8PC, 5 = grouped Q4G32 with SwiGLU, N = gate rows, 6 = Q8G64 with
 * the argmax epilogue, 7 = Q8G128 with the argmax epilogue, 8/9/10 = the
 * matrix-core kernel for Q8G64/Q8G128/Q8PC, named "<fmt>_mma_m<m>", 11 =
 * the matrix-core kernel for Q4G32, "q4g32_mma_m<m>").
 * Returns QG_OK or the status the call itself would return for that shape. */
qg_status qg_variant_name(int fmt, int64_t m, int64_t N, int64_t K, char *buf, size_t buf_len);
/* Launch-geometry override for the per-shape launch sweeps of the vllm.cpp
 * pull request #1936 commit log (tile and work-group counts swept per shape,
 * a choice adopted only on measured evidence).
 * Overrides how the non-matrix-core kernels (qgemv_q8g64, qgemv_q4g32,
 * qgemv_q8g128, qgemv_q8pc, the grouped calls and the *_argmax calls) map
 * tiles to waves, for tests and tuning sweeps.  Every tile is computed the
 * same way under any mapping, so results are the same bits.
 *   target_waves  > 0: about this many waves per launch in total (capped at
 *                 one wave per tile); 0: the per-compute-unit default.
 *   contig        1: each wave streams a contiguous run of tiles; 0: waves
 *                 sweep the matrix grid-stride; -1: the default (contiguous
 *                 for grouped calls, grid-stride otherwise).
 *   ring_depth    2 or 4: work items kept in flight per wave, with the
 *                 activation rows staged in LDS; 1: each lane holds its own
 *                 units of x in registers and the ring holds one tile (for
 *                 m = 1 and layouts of 2, 3 or 5 steps per tile and at least
 *                 16 lanes per row; elsewhere the default); 0: default.
 * Process-wide and sticky until called again with (0, -1, 0).  The three
 * values are stored together atomically: a call on another host thread uses
 * either the old or the new geometry.  The environment variable
 * QG_FORCE_VARIANT ("waves=N,wpcu=N,contig=0|1,ring=2|4|xr", any subset),
 * read at every call, does the same with lower precedence; both take
 * precedence over the library's per-shape policy.  The same variable also
 * takes ksplit=1|4|16, xg=0|1, mmawaves=N, mmacu=N and mmaeven=0|1 for the
 * matrix-core kernels (K split, x read from memory or staged, the wave
 * count the split is chosen for, work-groups per CU and even rounds of a
 * split launch), n=N,k=K,m=M to force only calls of that shape, and policy=0
 * to leave out the per-shape policies.  The plain kernels compute each
 * output the same way under every choice (the same bits); a different
 * matrix-core K split changes how each output's partial sums are grouped
 * (its results stay within the same bar).
 * Returns QG_ERR_INVALID_ARG (and changes nothing) for values outside these
 * ranges or target_waves above 2^24. */
qg_status qg_set_launch_override(int64_t target_waves, int32_t contig, int32_t ring_depth);
/* Per-wave timeline, for diagnostics: off by default, into a buffer the
 * caller allocates once, with what does not fit dropped and counted (the
 * native profiler of the MetaInfer-cpp README, section "M6 Reliability 与
 * Performance Evidence").
 * With device_records set, every launch with one activation row (m = 1) of
 * the non-matrix-core kernels (qgemv_q8g64, qgemv_q4g32, qgemv_q8g128,
 * qgemv_q8pc, the grouped calls and the *_argmax calls) runs a traced copy
 * of its kernel (the untraced kernels carry no trace code) and reserves one
 * record per wave in the buffer, launch after launch; each wave writes its
 * record as it ends: eight uint64
 * values, [0] start (the wave has its arguments and, in grouped calls, its
 * expert id, and is about to issue its first weight loads), [1] first
 * weights in (0 where the wave streamed nothing), [2] end, all in ticks of
 * the GPU's constant 100 MHz clock
 * (s_memrealtime), [3] the hardware id register (compute unit, SIMD, shader
 * engine), [4] the XCC (XCD) id, [5] slot, [6] wave index in the slot, [7]
 * the launch's index since the buffer was set.  Record i of a launch of W
 * waves per slot is slot * W + wave.  A launch whose waves do not fit in
 * the space left is not traced and counts as dropped.
 *   device_records     device memory, 8-byte aligned, capacity_records * 64
 *                      bytes, owned by the caller and kept alive while
 *                      traced launches may run; NULL turns tracing off.
 *   capacity_records   > 0 with a buffer.
 * Setting a buffer (or NULL) restarts the count.  Process-wide; launches on
 * several streams at once share the buffer in the order they are enqueued.
 * The records are valid once the traced launches have completed.
 * qg_wave_trace_state reports the records reserved, the launches traced and
 * the launches dropped since the buffer was set.
 * Returns QG_ERR_INVALID_ARG for a misaligned buffer or a capacity <= 0
 * with a buffer (changing nothing), or for NULL outputs. */
qg_status qg_set_wave_trace(void *device_records, int64_t capacity_records);
qg_status qg_wave_trace_state(int64_t *records, int64_t *launches, int64_t *dropped);

/* ------------------------------------------------------ measurement hook
 * A plain read of `bytes` bytes at buf (device, 16-byte aligned, bytes a
 * nonzero multiple of 16) with the GEMV kernels' access width: 16-byte
 * non-temporal loads, a wave-wide load one contiguous KiB, each wave
 * reading 8 KiB chunks (eight loads in flight, lane l taking units l,
 * l + 64, ... of the chunk) and the waves taking chunks grid-stride.  It is the bandwidth reference that a
 * weight-streaming call is compared with on the same part (effective weight
 * bandwidth over the bandwidth of a read of the same bytes; the zLLM post
 * defines effective bandwidth as bytes over kernel time).
 * Each lane XOR-folds the 32-bit words of the units it reads (word by word,
 * then the four words together); a lane whose fold is 0x9E3779B9 writes that
 * value to *sink (device, 4-byte aligned), so the loads cannot be dropped.
 * waves_per_cu: waves per compute unit, 1..32, or 0 for 8.  Asynchronous
 * on hip_stream (NULL = default stream).  QG_ERR_INVALID_ARG for a null
 * pointer, bytes 0 or not a multiple of 16, or waves_per_cu out of range;
 * QG_ERR_ALIGNMENT for a misaligned buf or sink; QG_ERR_HIP if the launch
 * fails.  Nothing is enqueued on error. */
qg_status qg_read_stream(const void *buf, size_t bytes, uint32_t *sink, int32_t waves_per_cu,
                         void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
