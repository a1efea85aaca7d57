// Host-side launch wrappers shared between the kernel translation units and
// the C ABI. Each returns the hipError_t of its launch; arguments are
// validated by the caller (h3dit_api.hip) before any of these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace h3 {

// Varlen bookkeeping (bookkeeping.hip)
size_t bookkeeping_scratch_bytes(int num_seqs);
// The schedule's per-segment query-tile prefix in work-list order (segments
// by descending length), num_seqs + 1 entries, inside that scratch; valid
// on the stream once launch_bookkeeping has written the list.
const int32_t* bookkeeping_rank_prefix(const void* scratch, int num_seqs);
hipError_t launch_bookkeeping(const int32_t* cu, int num_seqs, int total_tokens, int num_heads,
                              int block_m, int32_t* seg_id, int32_t* tile_cu, int32_t* items,
                              int64_t items_capacity, void* scratch, hipStream_t stream);

// bf16 flash attention over the work list (attn_bf16.hip)
hipError_t launch_attn_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            uint16_t* o, int64_t qs, int64_t ks, int64_t vs, int64_t os,
                            const int32_t* cu, const int32_t* items, int64_t num_items,
                            int num_seqs, int total_tokens, int num_heads, int head_dim,
                            float softmax_scale, const int32_t* rank_prefix, hipStream_t stream);

// fp8 quantisation (fp8_quant.hip): Q/K block codes, V channel codes, scales
size_t fp8_tiles_upper_bound(int num_seqs, int total_tokens);
size_t fp8_quant_workspace_bytes(int num_seqs, int total_tokens, int num_heads);
hipError_t launch_fp8_quantize(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t qs,
                               int64_t ks, int64_t vs, const int32_t* cu, int num_seqs,
                               int num_heads, int64_t num_tiles, uint8_t* q8, uint8_t* k8,
                               uint8_t* v8t, float* qsc, float* ksc, float* vsc, void* workspace,
                               hipStream_t stream, int16_t* qsum = nullptr, int16_t* ksum = nullptr);

// fp8 attention over the quantised codes (attn_fp8.hip)
size_t fp8_scratch_bytes(int num_seqs, int total_tokens, int num_heads, int head_dim);
hipError_t launch_attn_fp8(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           uint16_t* o, int64_t qs, int64_t ks, int64_t vs, int64_t os,
                           const int32_t* cu, const int32_t* cu_host, const int32_t* items,
                           int64_t num_items, int num_seqs, int total_tokens, int num_heads,
                           int head_dim, float softmax_scale, int skip, float skip_threshold,
                           int32_t* skip_counts, void* scratch, const int32_t* rank_prefix,
                           hipStream_t stream);

// Block-sparse attention, INT8 Q/K + FP8 V (bsa_select.hip, attn_fp8.hip).
// Lists: int32 [H, T, list_stride], row (head, first 64-token block of a
// 256-row query block) holds the kept key blocks of that query block.
constexpr int kBsaMaxKeyBlocks = 4096;          // 64-key blocks per segment
hipError_t launch_bsa_select(const int16_t* qsum, const int16_t* ksum, const float* qsc, const float* ksc,
                             const int32_t* cu, const int32_t* tb, const int32_t* items, int64_t num_items,
                             int num_seqs, int total_tokens, int num_heads, int64_t num_tiles,
                             int sp_permille, int64_t list_stride, int32_t* lists, int max_key_blocks,
                             hipStream_t stream);
size_t bsa_scratch_bytes(int num_seqs, int total_tokens, int num_heads, int64_t list_stride);
hipError_t launch_attn_bsa(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           int64_t qs, int64_t ks, int64_t vs, int64_t os, const int32_t* cu,
                           const int32_t* cu_host, const int32_t* items, int64_t num_items,
                           int num_seqs, int total_tokens, int num_heads, float softmax_scale,
                           int sp_permille, int64_t list_stride, int32_t* lists_out, void* scratch,
                           const int32_t* rank_prefix, hipStream_t stream);

// Q/K RMSNorm + 3D RoPE (qk_norm_rope.hip)
hipError_t launch_qk_norm_rope(uint16_t* q, uint16_t* k, int64_t qs, int64_t ks,
                               const uint16_t* w_q, const uint16_t* w_k, const int32_t* grid,
                               int total_tokens, int num_heads, int head_dim,
                               const int32_t split[3], float theta, float eps,
                               hipStream_t stream);

// AdaLN: modulation GEMV and RMSNorm + modulate (adaln.hip)
hipError_t launch_modulation(const uint16_t* cond, const uint16_t* w_mod, float* mod,
                             int num_seqs, int hidden, hipStream_t stream);
hipError_t launch_adaln(const uint16_t* x, uint16_t* h, const float* shift, const float* scale,
                        int64_t mod_stride, const int32_t* cu, int num_seqs, int total_tokens,
                        int hidden, float eps, hipStream_t stream);

// GEMMs with epilogues (gemm.hip)
enum GemmEpilogue { kEpiStore = 0, kEpiSwiGLU = 1, kEpiGatedResidual = 2 };
hipError_t launch_gemm(int epilogue, const uint16_t* a, const uint16_t* w, const uint16_t* w2,
                       uint16_t* y, int64_t m, int64_t n, int64_t k, const uint16_t* res,
                       const float* gate, int64_t gate_stride, const int32_t* cu,
                       int num_seqs, hipStream_t stream);
// MXFP8 operands: E4M3 codes row-major [rows, k], E8M0 scales K-step-major
// (row r, block j at byte ((j / 4) rows + r) 4 + j % 4); y is bf16, or MXFP8
// (codes + y_sc) for the SwiGLU epilogue. k % 128 == 0.
hipError_t launch_adaln_mx(const uint16_t* x, uint8_t* h8, uint8_t* h_sc, const float* shift,
                           const float* scale, int64_t mod_stride, const int32_t* cu, int num_seqs,
                           int total_tokens, int hidden, float eps, hipStream_t stream);
hipError_t launch_frames_to_u8(const float* x, uint8_t* out, int64_t b, int c, int64_t pixels,
                               hipStream_t stream);
hipError_t launch_mx4_quantize(const uint16_t* x, int64_t ld, int64_t rows, int64_t k, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream);
hipError_t launch_gemm_mx4(int epilogue, const uint8_t* a, const uint8_t* a_sc, const uint8_t* w,
                           const uint8_t* w_sc, const uint8_t* w2, const uint8_t* w2_sc, void* y,
                           int64_t m, int64_t n, int64_t k, const uint16_t* res, const float* gate,
                           int64_t gate_stride, const int32_t* cu, int num_seqs, hipStream_t stream);
hipError_t launch_mx_quantize(const uint16_t* x, int64_t ld, int64_t rows, int64_t k, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream);
hipError_t launch_gemm_mx(int epilogue, const uint8_t* a, const uint8_t* a_sc, const uint8_t* w,
                          const uint8_t* w_sc, const uint8_t* w2, const uint8_t* w2_sc, void* y,
                          uint8_t* y_sc, int64_t m, int64_t n, int64_t k, const uint16_t* res,
                          const float* gate, int64_t gate_stride, const int32_t* cu, int num_seqs,
                          hipStream_t stream);

}  // namespace h3
