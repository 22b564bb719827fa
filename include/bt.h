/*
 * bt.h -- C ABI of the ternary-weight x INT8-activation matmul for AMD MI355X (gfx950).
 *
 * The operation ("VibeVoice-ASR-BitNet Technical Report", section 2.2.2): the
 * decoder's linear layers hold weights in {-1, 0, +1} stored in 2 bits, with one
 * fp32 scale per weight tensor; activations are quantized to INT8 online, per
 * token; the kernel unpacks the 2-bit codes to INT8 and runs an integer
 * multiply-add (section 2.4.2, Figure 4: each output is one weight row dotted
 * with the activation vector, summed exactly). The tiling is chosen at run time
 * from the matrix dimensions (section 2.4.2); here that is a GEMV for M <= 16
 * and an MFMA GEMM above.
 *
 * Conventions shared by every entry point:
 *   - Row-major throughout. Activations x / xq are M x K (K contiguous); the
 *     weight matrix W is N x K (row n feeds output n); y and acc are M x N.
 *   - The caller allocates and frees every buffer. The library allocates
 *     nothing, keeps no mutable global state, and may be called from several
 *     host threads.
 *   - "host" pointers are ordinary CPU memory and the call is synchronous.
 *     "device" pointers are GPU memory (hipMalloc or a torch CUDA tensor); such
 *     calls are enqueued on `stream` and return before the GPU work runs.
 *   - Arguments are validated on the host before anything is launched. On an
 *     error nothing is launched and no output is written. Launch failures are
 *     reported as BT_ERR_DEVICE.
 *   - Device pointers must be 16-byte aligned (BT_ERR_ALIGN otherwise).
 *   - Not checked on the device: x must be finite (NaN/Inf rows give
 *     unspecified results), and a repacked weight buffer must come from
 *     bt_repack_ternary with the same N and K.
 */
#ifndef BT_H
#define BT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bt_status {
    BT_OK = 0,
    BT_ERR_NULL = 1,       /* a required pointer is NULL                            */
    BT_ERR_SHAPE = 2,      /* M, N or K < 1, K % 128 != 0, K > BT_MAX_K, or a size
                              that overflows                                         */
    BT_ERR_VALUE = 3,      /* a weight outside {-1,0,1}, a 2-bit code 3, a bad scale */
    BT_ERR_ALIGN = 4,      /* a device pointer not 16-byte aligned                   */
    BT_ERR_DEVICE = 5,     /* the HIP runtime reported an error                      */
    BT_ERR_WORKSPACE = 6   /* workspace missing or smaller than required             */
} bt_status;

/* Elements per packed group along K (blog post "Paper 說支援 ARM，我大概是第一個真的
 * 去編譯的人", second postscript: the weight file stores codes in 128-element groups). */
#define BT_GROUP_K 128
/* Largest token count served by the GEMV path; larger M uses the MFMA GEMM. */
#define BT_GEMV_MAX_M 16
/* Largest K of the ternary format and matmul (a multiple of BT_GROUP_K).
 * |acc| <= 127 * K then stays below 2^24: every accumulator is exact in int32
 * and converts to fp32 exactly, and the kernels' 32-bit buffer offsets (128
 * token rows of K int8 per tile) cannot wrap. Larger K is BT_ERR_SHAPE. */
#define BT_MAX_K 131072

/* Human-readable name of a status code (static string, never NULL). */
const char* bt_status_string(bt_status status);

/* ---------------------------------------------------------------------------
 * Canonical packed format (host, synchronous).
 *
 * Technical report section 2.2.2: ternary weights in 2 bits; the blog post's
 * second postscript: 128-element groups, interleaved so that the decoding
 * depends on the group size. Code of a weight = w + 1 (-1 -> 0, 0 -> 1, +1 -> 2;
 * code 3 is invalid). Row n occupies K/4 bytes; byte 32g + b of the row holds
 * the elements 128g + 32s + b at bits 2s..2s+1, s = 0..3.
 * ------------------------------------------------------------------------- */

/* N*K/4 (one eighth of the FP16 matrix), or 0 if N < 1, K < 1, K % 128 != 0 or
 * K > BT_MAX_K. */
size_t bt_packed_bytes(int64_t N, int64_t K);

/* Pack w (host, N x K int8, values in {-1,0,1}) into packed (host, N*K/4 bytes).
 * BT_ERR_VALUE if any weight is outside {-1,0,1}; packed is then left untouched. */
bt_status bt_pack_ternary(const int8_t* w, int64_t N, int64_t K, uint8_t* packed);

/* Inverse of bt_pack_ternary (host). BT_ERR_VALUE if any 2-bit field is 3. */
bt_status bt_unpack_ternary(const uint8_t* packed, int64_t N, int64_t K, int8_t* w);

/* ---------------------------------------------------------------------------
 * Offline ternarization (device, once per weight tensor, before packing).
 *
 * Technical report section 2.2.2: the weights are quantized to ternary
 * following the BitNet approach of its reference [11] ("The era of 1-bit
 * LLMs"): the absmean quantizer. Over the whole N x K tensor, with
 * S = sum |w| taken in fp64 (any summation order):
 *   gamma = fl32(S / (N*K)) (the division in fp64); delta = fl32(gamma + eps);
 *   t = w / delta (IEEE fp32 division);
 *   w~ = clamp(round_half_away_from_zero(t), -1, 1), i.e. +-1 where |t| >= 1/2.
 * The codes are written in the canonical packed format above (as
 * bt_pack_ternary would pack w~) and gamma, the per-tensor scale that
 * multiplies them back, to *scale. delta == 0 (an all-zero tensor with
 * eps == 0) gives all-zero weights and gamma = 0.
 *
 * w: device fp32 N x K, finite (not checked). packed: device,
 * bt_packed_bytes(N,K) bytes, written. scale: device fp32 [1], written.
 * eps: finite and >= 0 (BT_ERR_VALUE otherwise). workspace: device, at least
 * bt_ternarize_workspace_bytes(N,K) bytes (per-workgroup partial sums; its
 * contents on entry do not matter). None of the four buffers may overlap
 * another (BT_ERR_VALUE). Two launches on `stream`; deterministic.
 * ------------------------------------------------------------------------- */
size_t bt_ternarize_workspace_bytes(int64_t N, int64_t K);
bt_status bt_ternarize(const float* w, int64_t N, int64_t K, float eps, uint8_t* packed,
                       float* scale, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* The same ternarization for many tensors (a model's weights at conversion
 * time), two launches in all instead of two per tensor: every tensor's
 * packed bytes and scale equal bt_ternarize's for it, bit for bit. A plan is
 * built on the host, copied by the caller into device memory (same bytes),
 * and launched any number of times: plan_host sizes the grids, plan_dev is
 * read by the kernels. Each descriptor obeys bt_ternarize's rules, with a
 * slice of the plan's workspace of bt_ternarize_workspace_bytes(N,K) bytes;
 * in addition no tensor's packed bytes or scale may overlap another tensor's
 * w, packed bytes or scale (BT_ERR_VALUE). Every check runs before the plan is
 * written. */
typedef struct bt_ternarize_desc {
    const float* w;     /* device fp32 N x K */
    int64_t N, K;
    float eps;
    uint8_t* packed;    /* device, bt_packed_bytes(N,K) bytes, written */
    float* scale;       /* device fp32 [1], written */
} bt_ternarize_desc;

size_t bt_ternarize_plan_bytes(int32_t count);
/* Sum of bt_ternarize_workspace_bytes over the descriptors (0 if one is invalid). */
size_t bt_ternarize_plan_workspace_bytes(const bt_ternarize_desc* descs, int32_t count);
/* workspace: device, at least bt_ternarize_plan_workspace_bytes bytes, owned
 * by the plan while it is in use (contents on entry do not matter). */
bt_status bt_ternarize_plan_build(const bt_ternarize_desc* descs, int32_t count,
                                  void* workspace, size_t workspace_bytes, void* plan_host,
                                  size_t plan_bytes);
bt_status bt_ternarize_grouped(const void* plan_host, const void* plan_dev, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Device repack (once per weight tensor, at load time).
 *
 * Permutes the canonical bytes into the kernels' fragment order: 16-row tiles,
 * each 16-element run of one row in one 32-bit word, 256-element steps stored
 * so that one 128-bit load per lane feeds four matrix-core steps. Rows are
 * padded to a multiple of 16 and K to a multiple of 256 (padding holds zero
 * weights). The layout is private to the library; only bt_ternary_matmul*
 * read it.
 * ------------------------------------------------------------------------- */

/* ceil(N/16)*16 * ceil(K/256)*256 / 4, or 0 for invalid N, K. */
size_t bt_repacked_bytes(int64_t N, int64_t K);

/* packed_dev: device, bt_packed_bytes(N,K) canonical bytes.
 * wdev: device, bt_repacked_bytes(N,K) bytes, written. Must not overlap packed_dev. */
bt_status bt_repack_ternary(const uint8_t* packed_dev, int64_t N, int64_t K, void* wdev,
                            hipStream_t stream);

/* The same repack for many tensors in one launch (a model's weights at load
 * time: one launch instead of one per tensor, which for the decoder's 112
 * tensors of 0.6-7 MB would otherwise be bound by launch gaps). A plan is
 * built on the host, copied by the caller into device memory (same bytes),
 * and launched: plan_host sizes the grid, plan_dev is read by the kernel.
 * Each descriptor obeys bt_repack_ternary's rules; errors are reported by
 * bt_repack_plan_build before anything is launched. */
typedef struct bt_repack_desc {
    const uint8_t* packed_dev;   /* device, bt_packed_bytes(N,K) canonical bytes */
    void* wdev;                  /* device, bt_repacked_bytes(N,K) bytes, written */
    int64_t N, K;
} bt_repack_desc;

size_t bt_repack_plan_bytes(int32_t count);
bt_status bt_repack_plan_build(const bt_repack_desc* descs, int32_t count, void* plan_host,
                               size_t plan_bytes);
bt_status bt_repack_ternary_grouped(const void* plan_host, const void* plan_dev,
                                    hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Per-token absmax INT8 quantization (technical report section 2.2.2:
 * activations quantized to INT8 online per token).
 *
 * Per row m, each step in IEEE fp32: a = max_k |x[m,k]|; inv = 127 / a
 * (correctly rounded); q = clamp(round_half_away_from_zero(x * inv), -127, 127);
 * xscale[m] = a / 127; xsum[m] = sum_k q[m,k]. A row with a == 0, or whose
 * 127 / a overflows, gives q = 0, xscale = 0, xsum = 0.
 *
 * x: device fp32 M x K. xq: device int8 M x K. xscale: device fp32 [M].
 * xsum: device int32 [M], may be NULL. K need not be a multiple of 128.
 * ------------------------------------------------------------------------- */
bt_status bt_quantize_act(const float* x, int64_t M, int64_t K, int8_t* xq, float* xscale,
                          int32_t* xsum, hipStream_t stream);

/* RMS normalization with a per-channel scale fused with the quantization above
 * ("VibeVoice-ASR-BitNet Technical Report" section 2.4.1: rms_norm_scaled, an
 * RMS normalization with a scale parameter; section 2.2.2: INT8 activations
 * per token). Per row m, with S = sum_k x[m,k]^2 taken in fp64 (each square is
 * exact; any summation order):
 *   ms = fl32(S / K); r = fl32(1 / fl32(sqrt(fl32(ms + eps)))), or r = 0 if
 *   that is not finite; h[k] = fl32(fl32(x[m,k] * r) * g[k]);
 * then h is quantized exactly as bt_quantize_act quantizes x (q, d, row sum).
 * h itself is not written. x: device fp32 M x K; g: device fp32 [K]; eps: fp32,
 * finite and >= 0 (BT_ERR_VALUE otherwise); xq, xscale, xsum as in
 * bt_quantize_act. Same shape and alignment rules as bt_quantize_act. */
bt_status bt_rmsnorm_quantize(const float* x, const float* g, float eps, int64_t M, int64_t K,
                              int8_t* xq, float* xscale, int32_t* xsum, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Ternary matmul with fp32 rescale (technical report section 2.4.2, Figure 4).
 *
 * acc[m,n] = sum_k xq[m,k] * w[n,k]   (exact int32; |acc| <= 127*K)
 * y[m,n]   = fl32( fl32(acc[m,n]) * fl32(xscale[m] * w_scale) )
 *
 * xq, xscale, xsum: as written by bt_quantize_act (xsum is required: the
 *   kernels multiply by the codes w+1 and subtract xsum).
 * wdev: bt_repack_ternary output for this N, K.
 * y: device fp32 M x N, written. acc: device int32 M x N or NULL.
 * workspace: device, at least bt_matmul_workspace_bytes(M,N,K) bytes (may be
 *   NULL when that is 0); its contents on entry do not matter. A shape needs
 *   one when its K is split: GEMVs (M <= 16) whose M x K int8 activations do
 *   not fit one workgroup's LDS slice, and GEMMs with fewer output tiles than
 *   compute units and a K long enough for the split to pay (the library's
 *   choice, made from M, N, K alone). Each K range writes its int32 partial
 *   sums to a slice of its own, and a second launch adds the slices in a fixed
 *   order (exact) and applies the scales and the epilogue. Calls that share
 *   one workspace must be ordered on one stream.
 * w_scale must be finite (BT_ERR_VALUE otherwise).
 * ------------------------------------------------------------------------- */
size_t bt_matmul_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Quantization fused into the GEMV (M <= BT_GEMV_MAX_M): the same result as
 * bt_quantize_act followed by bt_ternary_matmul, in one launch. Every
 * workgroup quantizes the whole of each token row (the row sums and scales
 * need all of it) and keeps its own K range, so it pays off for small M (the
 * decode step). x: device fp32 M x K. xq, xscale, xsum: optional outputs
 * (NULL to skip), written with exactly bt_quantize_act's values. Workspace as
 * for bt_ternary_matmul with the same M, N, K. */
bt_status bt_ternary_matmul_fused(int64_t M, int64_t N, int64_t K, const float* x,
                                  const void* wdev, float w_scale, float* y, int32_t* acc,
                                  int8_t* xq, float* xscale, int32_t* xsum, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

bt_status bt_ternary_matmul(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                            const float* xscale, const int32_t* xsum, const void* wdev,
                            float w_scale, float* y, int32_t* acc, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation and arguments as bt_ternary_matmul without the workspace. Where
 * the shape splits K, the partial sums go to a fixed array of
 * BT_NOALLOC_SCRATCH_BYTES inside the library; every GPU the library runs on
 * holds its own copy of it until the process ends, and its address is looked
 * up (hipGetSymbolAddress, once per device) on the first call that needs it.
 * The call itself allocates nothing (no hipMalloc, hipFree or allocating
 * library routine). A shape whose bt_matmul_workspace_bytes(M,N,K) exceeds
 * BT_NOALLOC_SCRATCH_BYTES returns BT_ERR_WORKSPACE before anything is
 * launched. The array's contents on entry do not matter (each K range writes
 * its whole slice before it is read), but all calls on one GPU share it:
 * calls that may run at the same time on one GPU (unordered streams) race,
 * so order them on one stream or with events. */
#define BT_NOALLOC_SCRATCH_BYTES (16u << 20)
bt_status bt_ternary_matmul_noalloc(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                                    const float* xscale, const int32_t* xsum, const void* wdev,
                                    float w_scale, float* y, int32_t* acc, hipStream_t stream);

/* The fused epilogues of the technical report's section 2.4.1 on the output
 * ("mul_mat_add_relu": matrix multiply + bias + ReLU; "add_scaled": residual
 * addition with layer-scale multiplication). With y the plain output above,
 * each step one fp32 operation and each optional:
 *   y1 = fl32(y + bias[n]);  y2 = relu ? (y1 > 0 ? y1 : +0) : y1;
 *   y3 = fl32(layer_scale[n] * y2);  out[m,n] = fl32(residual[m,n] + y3).
 * acc, when requested, is still the plain int32 sum. bias and layer_scale are
 * device fp32 [N], residual device fp32 M x N (row-major); each may be NULL and
 * must be 16-byte aligned. residual may be y itself (an in-place residual
 * update) but must not partly overlap it (BT_ERR_VALUE). */
typedef struct bt_epilogue {
    const float* bias;
    const float* layer_scale;
    const float* residual;
    int32_t relu;
    int32_t reserved;       /* set to 0 */
} bt_epilogue;

/* bt_ternary_matmul followed by the epilogue *epi (host memory; NULL = none). */
bt_status bt_ternary_matmul_epilogue(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                                     const float* xscale, const int32_t* xsum, const void* wdev,
                                     float w_scale, const bt_epilogue* epi, float* y,
                                     int32_t* acc, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* ---------------------------------------------------------------------------
 * I8_S: int8 weights x int8 activations ("VibeVoice-ASR-BitNet Technical
 * Report" section 2.2.1: the tokenizer's INT8 datapath; section 2.4.2 and
 * Figure 4: one integer multiply-add pipeline shared with I2_S, which only
 * adds the 2-bit unpack). acc[m,n] = sum_k xq[m,k] * w[n,k] exactly in int32,
 * y = fl32(fl32(acc) * fl32(xscale[m] * w_scale)), then the optional epilogue.
 * Weights are int8 over [-128, 127] with one fp32 scale per tensor;
 * activations come from bt_quantize_act (or bt_rmsnorm_quantize).
 * K % 32 == 0 and K <= 131072 (so that |acc| <= 127*128*K < 2^31).
 * ------------------------------------------------------------------------- */

/* ceil(N/16)*16 * ceil(K/256)*256, or 0 for invalid N, K. */
size_t bt_int8_repacked_bytes(int64_t N, int64_t K);

/* w_dev: device int8 N x K row-major. wdev: device, bt_int8_repacked_bytes
 * bytes, written (the kernels' tile order; padding holds zeros). */
bt_status bt_repack_int8(const int8_t* w_dev, int64_t N, int64_t K, void* wdev,
                         hipStream_t stream);

/* Workspace bt_int8_matmul needs for this shape (0 if none): shapes with too
 * few output tiles to fill the device split K, each K range writing its partial
 * sums to a slice of the workspace. Same rules as for bt_ternary_matmul's. */
size_t bt_int8_matmul_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* xq: device int8 M x K; xscale: device fp32 [M]; w8dev from bt_repack_int8;
 * epi: host, NULL for none (as bt_ternary_matmul_epilogue); acc may be NULL. */
bt_status bt_int8_matmul(int64_t M, int64_t N, int64_t K, const int8_t* xq, const float* xscale,
                         const void* w8dev, float w_scale, const bt_epilogue* epi, float* y,
                         int32_t* acc, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Grouped launches: many independent projections in one kernel launch.
 *
 * The technical report's kernels have "batch" tiling variants chosen by shape
 * (section 2.4.2); here a batch is a list of independent projections (for
 * example all 112 linear layers of one decode step when their inputs are
 * ready), so one launch keeps every compute unit streaming weights instead of
 * paying one launch per small matrix.
 *
 * A plan is built once on the host from descriptors, copied by the caller into
 * device memory (same bytes), and then launched any number of times. plan_host
 * and plan_dev must hold identical bytes; the host copy sizes the grid and the
 * device copy is read by the kernels. The buffers the descriptors point to must
 * stay valid while the plan is in use.
 * ------------------------------------------------------------------------- */
typedef struct bt_quant_desc {
    const float* x;   /* device fp32 M x K  */
    int8_t* xq;       /* device int8 M x K  */
    float* xscale;    /* device fp32 [M]    */
    int32_t* xsum;    /* device int32 [M]   (required in a grouped plan) */
    int64_t M, K;
} bt_quant_desc;

typedef struct bt_matmul_desc {
    int64_t M, N, K;        /* a plan holds GEMVs only (every M <= BT_GEMV_MAX_M) or
                               GEMMs only (every M > BT_GEMV_MAX_M, x NULL) */
    const int8_t* xq;       /* x == NULL: input from bt_quantize_act. x != NULL: optional output */
    const float* xscale;    /* same */
    const int32_t* xsum;    /* same */
    const void* wdev;
    float w_scale;
    float* y;
    int32_t* acc;           /* may be NULL */
    const float* x;         /* NULL, or fp32 M x K activations to quantize inside the launch
                               (then every descriptor of the plan must give x). Every
                               workgroup of a projection then quantizes all M rows itself:
                               that pays for a single token; a batch is faster quantized by
                               bt_quantize_act_grouped first (through the 28-layer decoder on
                               MI355X: 2 tokens 67 vs 69 us, 16 tokens 103 vs 278 us) */
} bt_matmul_desc;

size_t bt_quant_plan_bytes(int32_t count);
bt_status bt_quant_plan_build(const bt_quant_desc* descs, int32_t count, void* plan_host,
                              size_t plan_bytes);
bt_status bt_quantize_act_grouped(const void* plan_host, const void* plan_dev,
                                  hipStream_t stream);

size_t bt_matmul_plan_bytes(int32_t count);
/* Workspace the grouped launch of these descriptors needs (0 if none, or if a
 * descriptor is invalid). GEMVs: a projection whose M*K int8 activations do not
 * fit one workgroup's LDS slice is split along K, and its partial sums meet in
 * the workspace through atomics. GEMMs: a projection with fewer 128 x 256
 * output tiles than a quarter of the GPU's resident workgroups and a K of at
 * least 32 x 128 elements is split into K ranges of at most about 16 x 128; each range
 * stores its int32 partial sums in an M x N slice of the workspace, followed by
 * M int32 zeros. */
size_t bt_matmul_plan_workspace_bytes(const bt_matmul_desc* descs, int32_t count);
/* workspace: device memory of at least bt_matmul_plan_workspace_bytes bytes
 * (may be NULL when that is 0), zero-filled before its first use; it belongs
 * to the plan, and every completed launch leaves zero whatever a launch reads
 * as zero (GEMM slices are overwritten by each launch). BT_ERR_WORKSPACE if it
 * is missing or too small, BT_ERR_ALIGN if not 16-byte aligned; descriptors are
 * checked first and nothing is written to plan_host on an error. */
bt_status bt_matmul_plan_build(const bt_matmul_desc* descs, int32_t count, void* workspace,
                               size_t workspace_bytes, void* plan_host, size_t plan_bytes);
/* Every projection of the plan in one launch: GEMVs in one kernel (with the
 * quantization inside when the plan was built from x); GEMMs in one persistent
 * kernel, each projection on workgroup slots of its own, plus one launch per
 * split projection that adds its K ranges' partial sums and stores y (and acc).
 * Launches from one plan on one stream run in order; two streams launching the
 * same plan at once race on its workspace. */
bt_status bt_ternary_matmul_grouped(const void* plan_host, const void* plan_dev,
                                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BT_H */
