/*
 * h3dit.h - C ABI of the MI355X (gfx950) library for the packed joint
 * audio-video DiT hot path.
 *
 * The library computes one transformer block of a joint audio-video
 * diffusion transformer over a single packed token sequence: text, audio and
 * video tokens of each request sit back to back in one row, and only valid
 * tokens are ever computed (no padding). Sources, cited by page title and
 * section:
 *   [FastH3-EN] "MiniMax H3 FastH3 real-time serving with vLLM-Omni",
 *       section "System-wide optimizations in vLLM-Omni": the bullet on
 *       long-sequence attention (packed sequence, padding removed) and the
 *       bullet on fused DiT operators (RMSNorm, RoPE, modulation,
 *       normalization and SwiGLU fused into fewer launches); section
 *       "Scaling beyond the FastH3 profile", bullet on sparse & quantized
 *       attention (FP8 attention, Skip-Softmax).
 *   [FastH3-ZH] "FastH3 在八卡 B300 上实现完整 MP4 生成快于播放时长",
 *       sections "长序列注意力与通信优化" (about 58k packed tokens, valid
 *       tokens only) and "融合 DiT 算子" (Q/K norm merged with RoPE, SwiGLU
 *       replacing SiLU + multiply, residual connection).
 * The pages name the operators but not their equations; each entry point
 * states the definition it implements.
 *
 * Conventions for every entry point:
 *  - Tensors are row-major. "bf16" buffers hold IEEE bfloat16 bit patterns.
 *    Linear weights use the [out, in] layout (both GEMM operands are
 *    contiguous along the reduction axis).
 *  - Pointers named *_dev / device pointers must be device memory of the
 *    current HIP device; *_host pointers are host memory read synchronously
 *    during the call. The caller owns every buffer, including workspaces.
 *    The library never allocates, frees or synchronises: it validates the
 *    arguments on the host, enqueues kernels on `hip_stream` (a hipStream_t,
 *    NULL for the default stream) and returns.
 *  - All argument checks run before the first launch, so a non-OK status
 *    means nothing was enqueued (except H3_ERR_HIP, reported when a launch
 *    itself fails; later launches of that call are then not enqueued).
 *    Faults inside kernels surface at the caller's next synchronisation.
 *  - cu_seqlens (int32[num_seqs + 1]): cu[0] = 0, non-decreasing,
 *    cu[num_seqs] = total_tokens. Empty segments are allowed. The host copy
 *    is validated; the device copy must hold the same values.
 *  - Thread safety: the only library state is a thread-local error message.
 */
#ifndef H3DIT_H
#define H3DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define H3_API __attribute__((visibility("default")))
#else
#define H3_API
#endif

#define H3_ABI_VERSION 1

/* Largest number of packed segments accepted by one call. */
#define H3_MAX_SEGMENTS 65536
/* Query rows per attention work item (the tile of the work list). */
#define H3_ATTN_BLOCK_M 256
/* Tokens per fp8 Q/K scale block (aligned to each segment's start). */
#define H3_FP8_QK_BLOCK 64

typedef enum {
    H3_OK = 0,
    H3_ERR_INVALID_ARGUMENT = 1, /* malformed sizes, pointers or cu_seqlens */
    H3_ERR_UNSUPPORTED = 2,      /* well-formed but not implemented (e.g. head_dim) */
    H3_ERR_WORKSPACE_TOO_SMALL = 3,
    H3_ERR_HIP = 4               /* a HIP runtime call or launch failed */
} h3_status;

typedef enum { H3_ATTN_BF16 = 0, H3_ATTN_FP8_E4M3 = 1 } h3_attn_precision;

/* Status name, e.g. "H3_ERR_UNSUPPORTED". Never NULL. */
H3_API const char* h3_status_string(h3_status status);
/* Detail of the last non-OK status returned on the calling thread ("" if none). */
H3_API const char* h3_last_error_message(void);
H3_API int32_t h3_abi_version(void);

/* ------------------------------------------------------------------------
 * Varlen bookkeeping ([FastH3-EN] long-sequence attention bullet: only the
 * valid tokens of the packed sequence are scheduled).
 *
 * Work list of the attention kernels: one item per (head, segment, query
 * tile of block_m rows), item = int32[4] {head, segment, first query token
 * (absolute index), rows in the tile}. Order: segments by descending length
 * (ties: ascending segment index), then head ascending, then query tile
 * ascending. Empty segments contribute no item. Count = num_heads *
 * sum_s ceil(L_s / block_m).
 * ---------------------------------------------------------------------- */

/* Host builder. items_out may be NULL to query the count only; otherwise it
 * must hold `capacity` items (4 * capacity int32). count_out (required)
 * receives the count. block_m must be positive. */
H3_API h3_status h3_build_schedule_host(const int32_t* cu_seqlens_host, int32_t num_seqs,
                                        int32_t num_heads, int32_t block_m,
                                        int32_t* items_out, int64_t capacity,
                                        int64_t* count_out);

/* Device builder, the same list bit for bit, plus:
 *   seg_id_dev  int32[total_tokens]: segment of each token (may be NULL);
 *   tile_cu_dev int32[num_seqs + 1]: tile_cu[0] = 0, tile_cu[s + 1] =
 *               tile_cu[s] + ceil(L_s / block_m) in segment order (may be NULL).
 * items_dev must hold items_capacity >= count items. Needs a workspace of
 * h3_varlen_bookkeeping_workspace_size(num_seqs) bytes. */
H3_API size_t h3_varlen_bookkeeping_workspace_size(int32_t num_seqs);
H3_API h3_status h3_varlen_bookkeeping(const int32_t* cu_seqlens_dev,
                                       const int32_t* cu_seqlens_host, int32_t num_seqs,
                                       int32_t total_tokens, int32_t num_heads,
                                       int32_t block_m, int32_t* seg_id_dev,
                                       int32_t* tile_cu_dev, int32_t* items_dev,
                                       int64_t items_capacity, void* workspace,
                                       size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * Varlen joint attention ([FastH3-EN] long-sequence attention bullet;
 * [FastH3-ZH] long-sequence attention section).
 *
 * For every segment s and head h: O = softmax(Q K^T * scale) V over the
 * segment's tokens only (non-causal, nothing across segments), fp32
 * accumulation, softmax as exp(S - rowmax)/sum.
 * q, k, v, out: bf16, token t / head h / dim d at ptr[t * tok_stride + h *
 * head_dim + d] (strides in elements; heads contiguous inside a token).
 * head_dim must be 64 or 128 (H3_ERR_UNSUPPORTED otherwise).
 *
 * precision = H3_ATTN_FP8_E4M3 ([FastH3-EN] sparse & quantized attention
 * bullet; [FastH3-ZH] section "其他加速路径：有损但可控", SAGE and
 * Skip-Softmax) quantises Q and K to OCP e4m3 with one scale per (head,
 * 64-token block aligned to the segment start), V with one scale per
 * (segment, head, channel), runs Q K^T and P V on fp8 MFMA with P encoded
 * as e4m3(448 * p) and the softmax denominator the row sum of those encoded
 * values (summed on the matrix core; a sum of the unquantised p, the plainer
 * reading of the method, differs from it by about 2e-3 relative Frobenius
 * error), and, with skip_softmax set, skips exp and P V for a key
 * tile of 64 keys when every valid row of a 32-row query group has its tile
 * maximum more than skip_threshold (natural-log units) below its running
 * maximum (never the segment's first key tile). fp8 needs head_dim 128.
 * skip_counts (optional, device int32[items]) receives per work item the
 * number of skipped (32-row group, key tile) pairs; no atomics are used.
 * ---------------------------------------------------------------------- */
typedef struct {
    int32_t precision;       /* h3_attn_precision */
    int32_t skip_softmax;    /* fp8 only; 0 = off */
    float skip_threshold;    /* natural-log units; <= 0 means 8 */
    float softmax_scale;     /* 0 means 1 / sqrt(head_dim) */
    int32_t* skip_counts;    /* optional device int32[work items] */
} h3_attn_opts;

/* opts may be NULL (bf16, default scale). */
H3_API size_t h3_attn_varlen_workspace_size(int32_t num_seqs, int32_t total_tokens,
                                            int32_t num_heads, int32_t head_dim,
                                            const h3_attn_opts* opts);
/* Number of work items (the length skip_counts must have). */
H3_API h3_status h3_attn_varlen_num_items(const int32_t* cu_seqlens_host, int32_t num_seqs,
                                          int32_t num_heads, int64_t* count_out);
H3_API h3_status h3_attn_varlen(const void* q, const void* k, const void* v, void* out,
                                int64_t q_tok_stride, int64_t k_tok_stride,
                                int64_t v_tok_stride, int64_t o_tok_stride,
                                const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                                int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                                int32_t head_dim, const h3_attn_opts* opts, void* workspace,
                                size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * h3_attn_varlen without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same computation, arguments,
 * layouts, validation and errors as h3_attn_varlen (bf16 or fp8, skip
 * options, skip_counts); the work list, the bookkeeping scratch and the fp8
 * code buffers live in a library-owned device array of
 * H3_NOALLOC_SCRATCH_BYTES (64 MiB), one per GPU, reserved when the library
 * is loaded onto that GPU and held until the process ends. Nothing is
 * allocated or freed, by the library or any library it calls.
 *  - The array's device address is looked up once per device, on the first
 *    call made with that device current (hipGetSymbolAddress); the stream
 *    must belong to the current device.
 *  - A call that needs more scratch than the array holds (its need is
 *    h3_attn_varlen_workspace_size for the same arguments: bf16 fits any
 *    size the other limits allow up to about 4 million work items; fp8 fits
 *    while N x H stays below about 170,000 token-heads) returns
 *    H3_ERR_WORKSPACE_TOO_SMALL before any launch.
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents (nothing in it needs to start at zero: every word a
 *    call reads, that call writes first). Calls ordered on one stream are
 *    safe; calls that overlap in time on one GPU (other streams, other
 *    threads without ordering) race on the array.
 * ---------------------------------------------------------------------- */
#define H3_NOALLOC_SCRATCH_BYTES (64u << 20)
H3_API h3_status h3_attn_varlen_noalloc(const void* q, const void* k, const void* v, void* out,
                                        int64_t q_tok_stride, int64_t k_tok_stride,
                                        int64_t v_tok_stride, int64_t o_tok_stride,
                                        const int32_t* cu_seqlens_dev,
                                        const int32_t* cu_seqlens_host, int32_t num_seqs,
                                        int32_t total_tokens, int32_t num_heads,
                                        int32_t head_dim, const h3_attn_opts* opts,
                                        void* hip_stream);

/* ------------------------------------------------------------------------
 * fp8 quantisation of Q, K and V, the first step of the fp8 attention path
 * ([FastH3-EN] sparse & quantized attention bullet; [FastH3-ZH] section
 * "其他加速路径：有损但可控": SAGE runs the attention computation in FP8).
 * h3_attn_varlen with H3_ATTN_FP8_E4M3 runs it internally; it is exported so
 * the codes can be inspected and reused.
 *
 * Format OCP e4m3fn (max 448). scale = amax / 448 stored as the fp32
 * quotient (1 when amax == 0); code = round-to-nearest-even(448 x / amax) of
 * the exact quotient (not of x divided by the rounded scale, which can move
 * an exact midpoint off the tie), saturating at +-448; 0 when amax == 0. Q and K: one scale per (64-token block aligned to the segment
 * start, head); V: one scale per (segment, head, channel). head_dim must be
 * 128. q, k, v as for h3_attn_varlen (bf16, token strides in elements,
 * multiples of 8, 16-byte aligned). T = sum over segments of ceil(L_s / 64)
 * (h3_fp8_num_tiles); block j of segment s is tile tile_cu64[s] + j.
 * Outputs (device, caller-owned):
 *   q8      uint8 [total_tokens, num_heads, 128], token-major;
 *   k8      uint8 [num_heads, T, 64, 128]: 64-token key tiles, rows past a
 *           segment's end are 0;
 *   v8t     uint8 [num_heads, T, 128, 64]: V transposed per tile; key
 *           32b + 8i + 4g + e of a tile (b, g in {0, 1}; i, e in 0..3) is at
 *           position 32g + 16b + 4i + e of its 64-byte channel row;
 *   q_scale, k_scale float [T, num_heads]; v_scale float [num_seqs,
 *           num_heads, 128].
 * Needs a workspace of h3_fp8_quantize_workspace_size(...) bytes.
 * ---------------------------------------------------------------------- */
H3_API h3_status h3_fp8_num_tiles(const int32_t* cu_seqlens_host, int32_t num_seqs,
                                  int64_t* tiles_out);
H3_API size_t h3_fp8_quantize_workspace_size(int32_t num_seqs, int32_t total_tokens,
                                             int32_t num_heads);
H3_API h3_status h3_fp8_quantize(const void* q, const void* k, const void* v,
                                 int64_t q_tok_stride, int64_t k_tok_stride,
                                 int64_t v_tok_stride, const int32_t* cu_seqlens_dev,
                                 const int32_t* cu_seqlens_host, int32_t num_seqs,
                                 int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                                 void* q8, void* k8, void* v8t, float* q_scale,
                                 float* k_scale, float* v_scale, void* workspace,
                                 size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * Block-sparse varlen attention with INT8 Q/K and FP8 V ("MiniMax H3 on
 * Ascend 950PR / 950DT", section "Recommended lossy configuration (Ascend
 * 950PR / 950DT)": EQBSA, block-sparse attention with Q and K in INT8 and V
 * in FP8, sparsity 0.8; section "Tuning the EQBSA dense-fallback window":
 * whole denoising steps at the start and end run dense attention instead,
 * which is the caller's choice per call).
 *
 * The page gives the method's name, precisions and sparsity only; this
 * implements one reading of the rest:
 *  - Q and K: INT8, one scale per (head, 64-token block aligned to the
 *    segment start), scale = fp32(amax / 127) (1 if amax == 0), code =
 *    round-half-even(127 x / amax). V: e4m3 per (segment, head, channel) as
 *    in the fp8 path of h3_attn_varlen.
 *  - Query blocks of 256 rows and key blocks of 64 keys, aligned to the
 *    segment start. A query block keeps keep(n) = max(1, n - floor(n p /
 *    1000)) of its segment's n key blocks, p = round(1000 sparsity): those
 *    with the highest score_j = ((sum over its 64-row blocks b, ascending,
 *    of sq_b I_bj) sk_j) / n_j, I_bj the integer dot product of the INT8
 *    code sums of Q block b and key block j, sq/sk the scales, n_j the keys
 *    in block j, each step one float64 rounding in this order; equal scores
 *    go to the lower block index (this equals the ranking by the exact
 *    scores unless two scores at the keep boundary lie within float64
 *    rounding of each other).
 *  - Attention over the kept blocks only, in ascending order: S = (Q8 K8)
 *    sq sk scale, online softmax, P = e4m3(448 p), l the row sum of P
 *    (as in the fp8 attention: within about 2e-3 of a sum of unquantised p),
 *    O = (sum P V8) sv / (448 l); fp32 accumulation, bf16 output.
 * q, k, v, out, strides, cu_seqlens as for h3_attn_varlen; head_dim must be
 * 128; a segment may hold at most 4096 * 64 = 262144 tokens
 * (H3_ERR_UNSUPPORTED otherwise). sparsity in [0, 1) (0: every block kept,
 * the dense INT8/FP8 attention); softmax_scale 0 means 1 / sqrt(128).
 * kv_block_lists (optional, device int32 [num_heads, T, list_stride], T =
 * h3_fp8_num_tiles, list_stride = h3_attn_block_sparse_list_stride):
 * receives, for each head h and 256-row query block whose first 64-token
 * block is tile t, the kept key-block indices (within the segment) in
 * ascending order at [h, t, 0 .. keep); other entries are not written.
 * The workspace (h3_attn_block_sparse_workspace_size bytes, 256-byte
 * aligned) also holds the INT8 codes, code sums and, without
 * kv_block_lists, the lists. Errors leave out untouched.
 * ---------------------------------------------------------------------- */
H3_API h3_status h3_attn_block_sparse_list_stride(const int32_t* cu_seqlens_host, int32_t num_seqs,
                                                  float sparsity, int64_t* stride_out);
/* 0 for unsupported sizes (head_dim != 128, sparsity outside [0, 1)). */
H3_API size_t h3_attn_block_sparse_workspace_size(int32_t num_seqs, int32_t total_tokens,
                                                  int32_t num_heads, int32_t head_dim,
                                                  float sparsity);
H3_API h3_status h3_attn_block_sparse(const void* q, const void* k, const void* v, void* out,
                                      int64_t q_tok_stride, int64_t k_tok_stride,
                                      int64_t v_tok_stride, int64_t o_tok_stride,
                                      const int32_t* cu_seqlens_dev,
                                      const int32_t* cu_seqlens_host, int32_t num_seqs,
                                      int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                                      float softmax_scale, float sparsity,
                                      int32_t* kv_block_lists, void* workspace,
                                      size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * Fused Q/K RMSNorm + 3D RoPE, in place ([FastH3-ZH] "融合 DiT 算子": the
 * Q/K normalisation is merged with RoPE).
 *
 * For every token t and head h, with x = q[t, h, :] (and likewise k):
 *   x <- RoPE_t(RMSNorm(x) * w),  RMSNorm(x) = x / sqrt(mean(x^2) + eps)
 * w_q / w_k: bf16 [head_dim] gains shared by all heads. RoPE: the head dim
 * is split into (d_t, d_h, d_w) = rope_split (even, summing to head_dim);
 * inside axis a's slice, pair j = dims (2j, 2j+1) is rotated by the angle
 * pos_a * theta^(-2j / d_a), (u, v) -> (u cos - v sin, u sin + v cos), with
 * pos = rope_grid[t] (device int32 [total_tokens, 3] = (t, h, w)).
 * q/k: bf16 with token strides in elements, heads contiguous. Math in fp32,
 * result rounded to bf16. head_dim 64 or 128.
 * ---------------------------------------------------------------------- */
H3_API h3_status h3_qk_rmsnorm_rope(void* q, void* k, int64_t q_tok_stride,
                                    int64_t k_tok_stride, const void* w_q, const void* w_k,
                                    const int32_t* rope_grid, int32_t total_tokens,
                                    int32_t num_heads, int32_t head_dim,
                                    const int32_t rope_split[3], float theta, float eps,
                                    void* hip_stream);

/* ------------------------------------------------------------------------
 * AdaLN modulation ([FastH3-EN] fused DiT operators bullet: modulation).
 *
 * mod[b, :] = cond[b, :] . W_mod^T (fp32 out, [num_seqs, 6 * hidden]);
 * cond bf16 [num_seqs, hidden], W_mod bf16 [6 * hidden, hidden]. The six
 * chunks of `hidden` are, in order: shift1, scale1, gate1, shift2, scale2,
 * gate2. fp32 accumulation.
 * ---------------------------------------------------------------------- */
H3_API h3_status h3_modulation(const void* cond, const void* w_mod, float* mod_out,
                               int32_t num_seqs, int32_t hidden, void* hip_stream);

/* RMSNorm + modulate ([FastH3-EN] fused DiT operators bullet: modulation and
 * normalization in one kernel):
 *   h[t, :] = RMSNorm(x[t, :]) * (1 + scale[seg(t), :]) + shift[seg(t), :]
 * x, h: bf16 [total_tokens, hidden] (row stride = hidden); shift, scale:
 * fp32 rows of `mod_row_stride` floats per segment (e.g. pointers into the
 * h3_modulation output, stride 6 * hidden). hidden must be a multiple of 512
 * and at most 8192. */
H3_API h3_status h3_adaln_rmsnorm_modulate(const void* x, void* h_out, const float* shift,
                                           const float* scale, int64_t mod_row_stride,
                                           const int32_t* cu_seqlens_dev,
                                           const int32_t* cu_seqlens_host, int32_t num_seqs,
                                           int32_t total_tokens, int32_t hidden, float eps,
                                           void* hip_stream);

/* ------------------------------------------------------------------------
 * Linear layers on bf16 MFMA with fused epilogues ([FastH3-ZH] "融合 DiT
 * 算子": SwiGLU in place of separate SiLU and multiply, the residual
 * connection; [FastH3-EN] fused DiT operators bullet).
 *
 * a: bf16 [m, k] (row stride k); weights bf16 [n, k]; output bf16 [m, n].
 * fp32 accumulation, one bf16 rounding at the end. m >= 0; n a multiple of
 * 8, k a multiple of 64. a and the weights 16-byte aligned, y and res 8-byte
 * aligned, gate 16-byte aligned with gate_row_stride a multiple of 4.
 *   h3_linear_bf16:              y = a . W^T
 *   h3_linear_swiglu_bf16:       y = silu(a . W_gate^T) * (a . W_up^T),
 *                                silu(z) = z / (1 + e^-z)
 *   h3_linear_gated_residual_bf16:
 *                                y[t, :] = res[t, :] + gate[seg(t), :] * (a . W^T)[t, :]
 *                                (res bf16 [m, n], may equal y; gate fp32 rows
 *                                of gate_row_stride floats per segment)
 * ---------------------------------------------------------------------- */
H3_API h3_status h3_linear_bf16(const void* a, const void* w, void* y, int64_t m, int64_t n,
                                int64_t k, void* hip_stream);
H3_API h3_status h3_linear_swiglu_bf16(const void* a, const void* w_gate, const void* w_up,
                                       void* y, int64_t m, int64_t n, int64_t k,
                                       void* hip_stream);
H3_API h3_status h3_linear_gated_residual_bf16(const void* a, const void* w, const void* res,
                                               const float* gate, int64_t gate_row_stride,
                                               void* y, int64_t m, int64_t n, int64_t k,
                                               const int32_t* cu_seqlens_dev,
                                               const int32_t* cu_seqlens_host,
                                               int32_t num_seqs, void* hip_stream);

/* ------------------------------------------------------------------------
 * Decoded frames to contiguous uint8 ([FastH3-ZH] "紧凑输出与并行 MP4 构建";
 * [FastH3-EN] system-wide optimizations, GPU output preparation bullet: the
 * decoder's FP32 BCTHW frames are converted once on the GPU to uint8
 * BTHWC). The pages give no value range or rounding; the map taken is the
 * decoded-video convention for [-1, 1], evaluated in fp32 in this order:
 *   out[b, t, h, w, c] = round_half_even(255 * clamp(x[b, c, t, h, w] * 0.5
 *                        + 0.5, 0, 1)),   NaN -> 0.
 * x: fp32 [batch, channels, frames, height, width] contiguous, 4-byte
 * aligned; out: uint8 [batch, frames, height, width, channels] contiguous.
 * channels <= 64; fastest when x and out are 16-byte aligned, channels <= 4
 * and frames * height * width is a multiple of 16. Zero-sized dims are a
 * no-op.
 * ---------------------------------------------------------------------- */
H3_API h3_status h3_frames_to_uint8_bthwc(const float* x, void* out, int64_t batch, int64_t channels,
                                          int64_t frames, int64_t height, int64_t width,
                                          void* hip_stream);

/* ------------------------------------------------------------------------
 * MXFP8 linears ([H3-950PR] "Recommended lossy configuration": the
 * transformer runs with MXFP8 online quantization; [FastH3-EN] "Scaling
 * beyond the FastH3 profile", quantization-paths bullet: online FP8 for the
 * linears). The pages do not give the format; this follows the public OCP
 * Microscaling (MX) v1.0 specification, MXFP8 with E4M3 elements:
 *   - blocks of 32 consecutive elements along k share one E8M0 scale
 *     (byte e means 2^(e - 127)); the scale of a block is
 *     2^(floor(log2 amax) - 8), never below 2^-127 (byte 0 for all-zero
 *     blocks);
 *   - elements are E4M3(x / scale), round to nearest even, saturating at
 *     +-448; the value of an element is scale * code.
 * An MX matrix [rows, k] is two buffers: codes, uint8 [rows, k] row-major,
 * and scales in K-step-major order, the scale of row r and block j
 * (elements 32j .. 32j+31) at byte ((j / 4) * rows + r) * 4 + j % 4
 * (rows * k / 32 bytes; the four scales of a row for one 128-element K step
 * form one aligned dword). k is a multiple of 128; codes are 16-byte and
 * scales 4-byte aligned; rows * k / 32 < 2^31.
 *
 *   h3_mx_quantize_bf16: bf16 x [rows, k] (row stride x_row_stride elements,
 *       >= k and a multiple of 8, x 16-byte aligned) -> MX codes + scales.
 *       Exact: equal to the definition above for every bf16 input.
 *   h3_linear_mxfp8: y = dq(a) . dq(W)^T, y bf16 [m, n] (8-byte aligned),
 *       a MX [m, k], W MX [n, k]; n a multiple of 8. fp32 accumulation in
 *       the matrix core, one bf16 rounding.
 *   h3_linear_swiglu_mxfp8: y = MX(silu(dq(a) . dq(W_gate)^T) * (dq(a) .
 *       dq(W_up)^T)): the product is quantised from fp32 (no bf16 step) into
 *       MX codes y [m, n] and y_scales (rows = m); n a multiple of 128.
 *   h3_linear_gated_residual_mxfp8: y = res + gate[seg(t)] * (dq(a) .
 *       dq(W)^T), as h3_linear_gated_residual_bf16 (res, y bf16 8-byte
 *       aligned; gate 16-byte aligned).
 * Errors as for the bf16 linears; all buffers are the caller's, nothing is
 * allocated and every launch goes on hip_stream.
 * ---------------------------------------------------------------------- */
/* The AdaLN RMSNorm + modulate of h3_adaln_rmsnorm_modulate with MXFP8
 * output: h is quantised from its fp32 values (no bf16 step) into codes
 * [total_tokens, hidden] and scales (rows = total_tokens). Arguments and
 * errors otherwise as there; codes 16-byte, scales 4-byte aligned. */
H3_API h3_status h3_adaln_rmsnorm_modulate_mxfp8(const void* x, void* h_codes, void* h_scales,
                                                 const float* shift, const float* scale,
                                                 int64_t mod_row_stride,
                                                 const int32_t* cu_seqlens_dev,
                                                 const int32_t* cu_seqlens_host, int32_t num_seqs,
                                                 int32_t total_tokens, int32_t hidden, float eps,
                                                 void* hip_stream);
H3_API h3_status h3_mx_quantize_bf16(const void* x, int64_t x_row_stride, int64_t rows, int64_t k,
                                     void* codes, void* scales, void* hip_stream);
H3_API h3_status h3_linear_mxfp8(const void* a, const void* a_scales, const void* w,
                                 const void* w_scales, void* y, int64_t m, int64_t n, int64_t k,
                                 void* hip_stream);
H3_API h3_status h3_linear_swiglu_mxfp8(const void* a, const void* a_scales, const void* w_gate,
                                        const void* w_gate_scales, const void* w_up,
                                        const void* w_up_scales, void* y, void* y_scales, int64_t m,
                                        int64_t n, int64_t k, void* hip_stream);
H3_API h3_status h3_linear_gated_residual_mxfp8(const void* a, const void* a_scales, const void* w,
                                                const void* w_scales, const void* res,
                                                const float* gate, int64_t gate_row_stride, void* y,
                                                int64_t m, int64_t n, int64_t k,
                                                const int32_t* cu_seqlens_dev,
                                                const int32_t* cu_seqlens_host, int32_t num_seqs,
                                                void* hip_stream);

/* ------------------------------------------------------------------------
 * One DiT block over the packed sequence (all of the above, in order):
 *   mod = cond W_mod^T                      -> shift1 scale1 gate1 shift2 scale2 gate2
 *   h   = RMSNorm(x)(1 + scale1) + shift1
 *   qkv = h W_qkv^T                         (q | k | v, each [H * D], head-major)
 *   q,k = RoPE(RMSNorm_D(q|k) * gain)       (h3_qk_rmsnorm_rope)
 *   o   = varlen attention(q, k, v)         (bf16 path)
 *   x1  = x + gate1 * (o W_o^T)
 *   h2  = RMSNorm(x1)(1 + scale2) + shift2
 *   a   = silu(h2 W_gate^T) * (h2 W_up^T)
 *   x2  = x1 + gate2 * (a W_down^T)        -> x_out
 * This is a plain reading of the operator list of [FastH3-EN]'s fused DiT
 * operators bullet and [FastH3-ZH]'s "融合 DiT 算子" section as a
 * single-stream pre-norm AdaLN-Zero block; cond is one bf16 vector of
 * `hidden` per segment (request). Every intermediate is stored in bf16
 * (mod in fp32). x, x_out: bf16 [total_tokens, hidden] (may not alias).
 * hidden = num_heads * head_dim; ffn_dim a multiple of 64.
 * ---------------------------------------------------------------------- */
typedef struct {
    int32_t hidden, num_heads, head_dim, ffn_dim;
    int32_t rope_split[3];
    float rope_theta, eps;
} h3_dit_dims;

typedef struct {
    const void *w_mod, *w_qkv, *w_o, *q_norm, *k_norm, *w_gate, *w_up, *w_down;
} h3_dit_weights;

/* Optional caller buffers for intermediates; a non-NULL field replaces the
 * workspace buffer of that intermediate, so the caller can read it after the
 * call. mod: fp32 [B, 6C]; h, o, x1, h2: bf16 [N, C]; qkv: bf16 [N, 3C];
 * a: bf16 [N, ffn]. */
typedef struct {
    float* mod;
    void *h, *qkv, *o, *x1, *h2, *a;
} h3_dit_taps;

H3_API size_t h3_dit_block_workspace_size(const h3_dit_dims* dims, int32_t num_seqs,
                                          int32_t total_tokens);
H3_API h3_status h3_dit_block_forward(const void* x, void* x_out, const void* cond,
                                      const h3_dit_weights* weights, const h3_dit_dims* dims,
                                      const int32_t* cu_seqlens_dev,
                                      const int32_t* cu_seqlens_host, int32_t num_seqs,
                                      int32_t total_tokens, const int32_t* rope_grid,
                                      const h3_dit_taps* taps, void* workspace,
                                      size_t workspace_bytes, void* hip_stream);


/* ------------------------------------------------------------------------
 * The same block with MXFP8 linears ([H3-950PR] "Recommended lossy
 * configuration", MXFP8 online quantization of the transformer; format as
 * for h3_linear_mxfp8): the four linears take MX weights (quantised once by
 * the caller with h3_mx_quantize_bf16) and MX activations produced in the
 * previous kernel: h and h2 by the AdaLN kernel from its fp32 values, o by
 * h3_mx_quantize_bf16 from the bf16 attention output, a by the SwiGLU
 * epilogue from fp32. qkv, x1 and x_out stay bf16; the modulation GEMV,
 * norms, RoPE and attention are the bf16 path's. ffn_dim a multiple of 128;
 * total_tokens * max(3 hidden, ffn_dim) / 32 < 2^31. Needs a workspace of
 * h3_dit_block_mx_workspace_size(...) bytes (256-byte aligned).
 * ---------------------------------------------------------------------- */
typedef struct {
    const void* codes;   /* E4M3 [rows, k] */
    const void* scales;  /* E8M0, K-step-major (see the MXFP8 linears) */
} h3_mx_matrix;
typedef struct {
    const void *w_mod, *q_norm, *k_norm;               /* bf16, as in h3_dit_weights */
    h3_mx_matrix w_qkv, w_o, w_gate, w_up, w_down;     /* MX, [out, in] */
} h3_dit_mx_weights;
H3_API size_t h3_dit_block_mx_workspace_size(const h3_dit_dims* dims, int32_t num_seqs,
                                             int32_t total_tokens);
H3_API h3_status h3_dit_block_forward_mxfp8(const void* x, void* x_out, const void* cond,
                                            const h3_dit_mx_weights* weights,
                                            const h3_dit_dims* dims,
                                            const int32_t* cu_seqlens_dev,
                                            const int32_t* cu_seqlens_host, int32_t num_seqs,
                                            int32_t total_tokens, const int32_t* rope_grid,
                                            void* workspace, size_t workspace_bytes,
                                            void* hip_stream);

/* ------------------------------------------------------------------------
 * The block in the pages' lossy configuration ("MiniMax H3 on Ascend 950PR
 * / 950DT", section "Recommended lossy configuration (Ascend 950PR /
 * 950DT)": EQBSA block-sparse attention together with MXFP8 online
 * quantisation of the transformer): h3_dit_block_forward_mxfp8 with its
 * attention step replaced by the block-sparse INT8/FP8 attention of
 * h3_attn_block_sparse at `sparsity` (default softmax scale). Arguments,
 * layouts and errors as for h3_dit_block_forward_mxfp8, plus those of
 * h3_attn_block_sparse (head_dim 128, segments of at most 262144 tokens,
 * sparsity in [0, 1)). The workspace (h3_dit_block_mx_bsa_workspace_size
 * bytes, 0 for unsupported sizes) replaces the dense attention's share with
 * the block-sparse pass's. The dense-fallback window of the pages (leading
 * and trailing denoising steps) is the caller's per-step choice between
 * this call and h3_dit_block_forward_mxfp8.
 * ---------------------------------------------------------------------- */
H3_API size_t h3_dit_block_mx_bsa_workspace_size(const h3_dit_dims* dims, int32_t num_seqs,
                                                 int32_t total_tokens, float sparsity);
H3_API h3_status h3_dit_block_forward_mxfp8_bsa(const void* x, void* x_out, const void* cond,
                                                const h3_dit_mx_weights* weights,
                                                const h3_dit_dims* dims,
                                                const int32_t* cu_seqlens_dev,
                                                const int32_t* cu_seqlens_host, int32_t num_seqs,
                                                int32_t total_tokens, const int32_t* rope_grid,
                                                float sparsity, void* workspace,
                                                size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * MXFP4 linears ([H3-950PR] section "MXFP4 online quantization": the DiT's
 * linears switch from MXFP8 to MXFP4 online quantisation; the pages give no
 * format). The OCP Microscaling (MX) v1.0 MXFP4 format with E2M1 elements:
 *   - blocks of 32 consecutive elements along k share one E8M0 scale
 *     2^(floor(log2 amax) - 2), never below 2^-127 (byte 0 for all-zero
 *     blocks);
 *   - elements are E2M1(x / scale): the nearest of 0, 0.5, 1, 1.5, 2, 3, 4,
 *     6 (index 0..7), a midpoint going to the even index, saturating at 6;
 *     the 4-bit code is index + 8 when x is negative (its sign bit, also
 *     where the value rounds to zero);
 *   - an MXFP4 matrix [rows, k] is codes, uint8 [rows, k / 2] (element 2i
 *     in the low nibble of byte i), and scales, rows * k / 32 bytes in
 *     K-step-major order with 8 bytes per row and 256-element K step: the
 *     scale of row r and block j at byte ((j / 8) * rows + r) * 8 +
 *     (j % 2) * 4 + (j % 8) / 2 (the step's even blocks in its first
 *     dword, the odd blocks in its second, the order in which the matrix
 *     core's lanes take them). k is a multiple of 256; codes are 16-byte and
 *     scales 8-byte aligned; rows * k / 32 < 2^31.
 *
 *   h3_mx4_quantize_bf16: bf16 x [rows, k] (row stride x_row_stride
 *       elements, >= k and a multiple of 8, x 16-byte aligned) -> MXFP4
 *       codes + scales, equal to the definition above for every bf16 input.
 *   h3_linear_mxfp4: y = dq(a) . dq(W)^T, y bf16 [m, n] (8-byte aligned),
 *       a MXFP4 [m, k], W MXFP4 [n, k]; n a multiple of 8; fp32 accumulation
 *       in the matrix core, one bf16 rounding.
 *   h3_linear_swiglu_mxfp4: y = silu(dq(a) . dq(W_gate)^T) * (dq(a) .
 *       dq(W_up)^T) in bf16 [m, n]; n a multiple of 128.
 *   h3_linear_gated_residual_mxfp4: y = res + gate[seg(t)] * (dq(a) .
 *       dq(W)^T), as h3_linear_gated_residual_bf16.
 * Errors as for the bf16 linears; all buffers are the caller's.
 * ---------------------------------------------------------------------- */
H3_API h3_status h3_mx4_quantize_bf16(const void* x, int64_t x_row_stride, int64_t rows, int64_t k,
                                      void* codes, void* scales, void* hip_stream);
H3_API h3_status h3_linear_mxfp4(const void* a, const void* a_scales, const void* w,
                                 const void* w_scales, void* y, int64_t m, int64_t n, int64_t k,
                                 void* hip_stream);
H3_API h3_status h3_linear_swiglu_mxfp4(const void* a, const void* a_scales, const void* w_gate,
                                        const void* w_gate_scales, const void* w_up,
                                        const void* w_up_scales, void* y, int64_t m, int64_t n,
                                        int64_t k, void* hip_stream);
H3_API h3_status h3_linear_gated_residual_mxfp4(const void* a, const void* a_scales, const void* w,
                                                const void* w_scales, const void* res,
                                                const float* gate, int64_t gate_row_stride, void* y,
                                                int64_t m, int64_t n, int64_t k,
                                                const int32_t* cu_seqlens_dev,
                                                const int32_t* cu_seqlens_host, int32_t num_seqs,
                                                void* hip_stream);

/* ------------------------------------------------------------------------
 * The block with MXFP4 linears ([H3-950PR] section "MXFP4 online
 * quantization"): as h3_dit_block_forward_mxfp8, with the five linear
 * weights given as MXFP4 matrices (h3_mx_matrix: codes and scales in the
 * MXFP4 layouts above, quantised once by the caller with
 * h3_mx4_quantize_bf16) and every activation that enters a linear (h, o,
 * h2, a) quantised to MXFP4 from its bf16 value by h3_mx4_quantize_bf16's
 * kernel. hidden and ffn_dim multiples of 256. Needs a workspace of
 * h3_dit_block_mx4_workspace_size(...) bytes (256-byte aligned; 0 for
 * unsupported dims).
 * ---------------------------------------------------------------------- */
H3_API size_t h3_dit_block_mx4_workspace_size(const h3_dit_dims* dims, int32_t num_seqs,
                                              int32_t total_tokens);
H3_API h3_status h3_dit_block_forward_mxfp4(const void* x, void* x_out, const void* cond,
                                            const h3_dit_mx_weights* weights,
                                            const h3_dit_dims* dims,
                                            const int32_t* cu_seqlens_dev,
                                            const int32_t* cu_seqlens_host, int32_t num_seqs,
                                            int32_t total_tokens, const int32_t* rope_grid,
                                            void* workspace, size_t workspace_bytes,
                                            void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* H3DIT_H */
