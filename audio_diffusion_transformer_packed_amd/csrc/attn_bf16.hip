// Padding-free varlen joint attention on bf16 MFMA (gfx950).
//
// Computes, per packed segment and head, O = softmax(Q K^T * scale) V over
// the segment's valid tokens only ("MiniMax H3 FastH3 real-time serving with
// vLLM-Omni", section "System-wide optimizations in vLLM-Omni", long-sequence
// attention bullet; "FastH3 在八卡 B300 上实现完整 MP4 生成快于播放时长",
// section "长序列注意力与通信优化").
//
// Design (CDNA4, 64-lane waves):
//  * one workgroup per work item (head, segment, 128-row query tile), four
//    waves of 32 query rows each; the work list comes from the bookkeeping
//    kernel, so no padded token is ever loaded or computed;
//  * the scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane then owns one query row (lane % 32)
//    and 16 of every 32 keys, so the row max and row sum are lane-local
//    apart from one exchange with the lane 32 away;
//  * O^T = V^T P^T: P stays in registers (converted to bf16 in the MFMA B
//    layout), V^T is read from LDS;
//  * K and V^T tiles of 64 keys are staged in LDS, double buffered, with the
//    next tile's global loads in flight during the current tile's math; one
//    barrier per key tile;
//  * online softmax in the exp2 domain, fp32 accumulation.
#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {
namespace {

constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 256;  // four waves

template <int D>
struct Lds {
    static constexpr int kStride = D + 8;        // K row: D dims + pad (bf16 elements)
    static constexpr int vStride = kBN + 8;      // V^T row: 64 keys + pad
    static constexpr int kElems = kBN * kStride;
    static constexpr int vElems = D * vStride;
    static constexpr int bufElems = kElems + vElems;
};

// One 64-key tile for one wave's 32 query rows: S^T = K Q^T, online softmax
// (lazy max, exp2 domain), O^T += V^T P^T. With MASK, keys at or past
// keys_left (the segment end) are excluded.
template <int D, bool MASK>
__device__ __forceinline__ void attn_tile(const uint16_t* __restrict__ kl,
                                          const uint16_t* __restrict__ vl,
                                          const bf16x8 (&qf)[D / 16], f32x16 (&oacc)[D / 32],
                                          float& m_run, float& l_run, float scale_log2,
                                          float lazy_raw, int keys_left, int l32, int g) {
    using L = Lds<D>;
    constexpr int KC = D / 16;
    constexpr int DB = D / 32;

    // S^T = K Q^T for keys [32b, 32b + 32) of the tile
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const u32x4 kf = *reinterpret_cast<const u32x4*>(kl + (32 * b + l32) * L::kStride + 16 * c + 8 * g);
            sacc[b] = mfma32x32x16(__builtin_bit_cast(bf16x8, kf), qf[c], sacc[b]);
        }
    }
    if (MASK) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 32 * b + 8 * (r >> 2) + 4 * g + (r & 3);
                if (key >= keys_left) sacc[b][r] = -INFINITY;
            }
    }

    float mt = sacc[0][0];
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, fmaxf(sacc[0][r], sacc[1][r]));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    if (__any(mt > m_run + lazy_raw)) {       // wave-uniform, rare after the first tiles
        // keeps this block a real branch (not if-converted into 64 multiplies
        // by a selected alpha on every tile)
        asm volatile("" ::: "memory");
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
    const float mb = m_run * scale_log2;

    float psum = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sacc[b][8 * t + e], scale_log2, -mb));
                psum += p;
                pf[b][t][e] = static_cast<__bf16>(p);
            }
        }
    }
    l_run += psum;

    // O^T += V^T P^T; k-step (b, t) covers keys 32b + 16t + [0, 16); lane half
    // g supplies keys 4g + [0,4) and 8 + 4g + [0,4) of it, the rows the S^T
    // accumulator gave this lane.
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const uint16_t* vrow = vl + (32 * db + l32) * L::vStride + 4 * g;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + 32 * b + 16 * t);
                const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 32 * b + 16 * t + 8);
                const u32x4 vf = {lo.x, lo.y, hi.x, hi.y};
                oacc[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, vf), pf[b][t], oacc[db]);
            }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, int64_t qs, int64_t ks,
    int64_t vs, int64_t os, const int32_t* __restrict__ cu, const int4* __restrict__ items,
    int num_seqs, int total_tokens, int num_heads, float scale_log2) {
    using L = Lds<D>;
    constexpr int KC = D / 16;                   // MFMA k-steps over the head dim
    constexpr int DB = D / 32;                   // 32-wide output blocks over the head dim
    constexpr int K_CHUNKS = kBN * D / 8;        // 16-byte chunks per K tile
    constexpr int K_PER_T = K_CHUNKS / kThreads; // per thread
    constexpr int V_GROUPS = (kBN / 4) * (D / 8);// (4 keys x 8 dims) groups per V tile
    static_assert(K_CHUNKS % kThreads == 0, "K tile split");
    static_assert(V_GROUPS <= kThreads, "V tile split");

    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * L::bufElems];

    const int4 it = items[blockIdx.x];
    const int head = it.x, seg = it.y, q0 = it.z, qlen = it.w;
    if (seg < 0 || seg >= num_seqs || head < 0 || head >= num_heads) return;
    const int kv0 = max(0, cu[seg]);
    const int kv1 = min(total_tokens, cu[seg + 1]);
    if (q0 < kv0 || qlen <= 0 || q0 + qlen > kv1) return;
    const int len = kv1 - kv0;
    const int ntiles = (len + kBN - 1) / kBN;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;

    // ---- Q fragment in registers (B operand of S^T = K Q^T) ----
    const int qrow_local = wave * 32 + l32;
    const bool qvalid = qrow_local < qlen;
    bf16x8 qf[KC];
    {
        const uint16_t* qp = q + static_cast<int64_t>(q0 + qrow_local) * qs +
                             static_cast<int64_t>(head) * D + 8 * g;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            const u32x4 ch = qvalid ? *reinterpret_cast<const u32x4*>(qp + 16 * c) : u32x4{0, 0, 0, 0};
            qf[c] = __builtin_bit_cast(bf16x8, ch);
        }
    }

    // ---- global -> register staging of one K/V tile ----
    // Every load is unconditional: rows past the segment end are clamped to
    // its last row (finite data of this segment); their scores are masked to
    // -inf in the last tile, so they contribute exactly zero.
    constexpr int K_ROWS_PER_PASS = kThreads / (D / 8);
    const int k_r0 = tid / (D / 8);
    const int k_c = tid % (D / 8);
    const int vg = tid;                          // V group of this thread
    const int v_key4 = vg % (kBN / 4);
    const int v_dchunk = vg / (kBN / 4);
    const bool v_active = vg < V_GROUPS;
    const uint16_t* kthr = k + static_cast<int64_t>(head) * D + 8 * k_c;
    const uint16_t* vthr = v + static_cast<int64_t>(head) * D + 8 * (v_active ? v_dchunk : 0);
    const int64_t k_pass_stride = static_cast<int64_t>(K_ROWS_PER_PASS) * ks;

    u32x4 kreg[K_PER_T];
    u32x4 vreg[4];

    f32x16 oacc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) oacc[b] = f32x16{};
    // Reference max of this lane's query row (raw score units). It only moves
    // when a tile's max exceeds it by more than kLazy / scale_log2, i.e. when
    // exp2 of a score relative to it would pass 2^kLazy; in between, p <= 2^kLazy
    // and O needs no rescale. The final O / l is the same softmax.
    constexpr float kLazy = 8.0f;
    const float lazy_raw = kLazy / scale_log2;
    float m_run = -INFINITY;
    float l_run = 0.f;         // partial row sum over this lane's keys

    // Loads of key tile `tile` into kreg / vreg (unconditional; see above).
#define H3_ATTN_LOAD_TILE(tile)                                                              \
    {                                                                                        \
        const int key0 = kv0 + (tile) * kBN;                                                 \
        if (key0 + kBN <= kv1) {                                                             \
            const uint16_t* kp = kthr + static_cast<int64_t>(key0 + k_r0) * ks;              \
            _Pragma("unroll") for (int i = 0; i < K_PER_T; ++i)                              \
                kreg[i] = *reinterpret_cast<const u32x4*>(kp + i * k_pass_stride);           \
            const uint16_t* vp = vthr + static_cast<int64_t>(key0 + 4 * v_key4) * vs;        \
            _Pragma("unroll") for (int r = 0; r < 4; ++r)                                    \
                vreg[r] = *reinterpret_cast<const u32x4*>(vp + r * vs);                      \
        } else {                                                                             \
            _Pragma("unroll") for (int i = 0; i < K_PER_T; ++i) {                            \
                const int key = min(key0 + k_r0 + i * K_ROWS_PER_PASS, kv1 - 1);             \
                kreg[i] = *reinterpret_cast<const u32x4*>(kthr + static_cast<int64_t>(key) * ks); \
            }                                                                                \
            _Pragma("unroll") for (int r = 0; r < 4; ++r) {                                  \
                const int key = min(key0 + 4 * v_key4 + r, kv1 - 1);                         \
                vreg[r] = *reinterpret_cast<const u32x4*>(vthr + static_cast<int64_t>(key) * vs); \
            }                                                                                \
        }                                                                                    \
    }

    // K rows as they are; V transposed to V^T[d][key] (4 keys x 8 dims per
    // thread: v_perm_b32 gathers the same dim of 4 keys into 8 bytes).
#define H3_ATTN_STORE_TILE(buf)                                                              \
    {                                                                                        \
        uint16_t* kl_ = lds + (buf) * L::bufElems;                                           \
        uint16_t* vl_ = kl_ + L::kElems;                                                     \
        _Pragma("unroll") for (int i = 0; i < K_PER_T; ++i)                                  \
            *reinterpret_cast<u32x4*>(kl_ + (k_r0 + i * K_ROWS_PER_PASS) * L::kStride + 8 * k_c) = kreg[i]; \
        if (v_active) {                                                                      \
            _Pragma("unroll") for (int w = 0; w < 4; ++w) {                                  \
                _Pragma("unroll") for (int hs = 0; hs < 2; ++hs) {                           \
                    const uint32_t sel = hs ? 0x07060302u : 0x05040100u;                     \
                    u32x2 t_;                                                                \
                    t_.x = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], sel);               \
                    t_.y = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], sel);               \
                    *reinterpret_cast<u32x2*>(vl_ + (8 * v_dchunk + 2 * w + hs) * L::vStride + 4 * v_key4) = t_; \
                }                                                                            \
            }                                                                                \
        }                                                                                    \
    }

    H3_ATTN_LOAD_TILE(0)
    H3_ATTN_STORE_TILE(0)
    __syncthreads();

    for (int tile = 0; tile + 1 < ntiles; ++tile) {
        H3_ATTN_LOAD_TILE(tile + 1)
        const uint16_t* kl = lds + (tile & 1) * L::bufElems;
        attn_tile<D, false>(kl, kl + L::kElems, qf, oacc, m_run, l_run, scale_log2, lazy_raw,
                            kBN, l32, g);
        H3_ATTN_STORE_TILE((tile & 1) ^ 1)
        __syncthreads();
    }
    {
        const int tile = ntiles - 1;
        const uint16_t* kl = lds + (tile & 1) * L::bufElems;
        const int keys_left = len - tile * kBN;
        if (keys_left < kBN)
            attn_tile<D, true>(kl, kl + L::kElems, qf, oacc, m_run, l_run, scale_log2, lazy_raw,
                               keys_left, l32, g);
        else
            attn_tile<D, false>(kl, kl + L::kElems, qf, oacc, m_run, l_run, scale_log2, lazy_raw,
                                kBN, l32, g);
    }
#undef H3_ATTN_LOAD_TILE
#undef H3_ATTN_STORE_TILE

    // ---- normalise and store ----
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.f / l_tot;
    if (qvalid) {
        uint16_t* op = o + static_cast<int64_t>(q0 + qrow_local) * os + static_cast<int64_t>(head) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = 32 * db + 8 * r4 + 4 * g;
                uint2 w;
                w.x = pack_bf16x2(oacc[db][4 * r4 + 0] * inv, oacc[db][4 * r4 + 1] * inv);
                w.y = pack_bf16x2(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv);
                *reinterpret_cast<uint2*>(op + d) = w;
            }
    }
}

}  // namespace

hipError_t launch_attn_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            uint16_t* o, int64_t qs, int64_t ks, int64_t vs, int64_t os,
                            const int32_t* cu, const int32_t* items, int64_t num_items,
                            int num_seqs, int total_tokens, int num_heads, int head_dim,
                            float softmax_scale, hipStream_t stream) {
    if (num_items <= 0) return hipSuccess;
    const float sl2 = softmax_scale * kLog2e;
    const dim3 grid(static_cast<unsigned>(num_items));
    if (head_dim == 128) {
        hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(kThreads), 0, stream, q, k, v, o, qs,
                           ks, vs, os, cu, reinterpret_cast<const int4*>(items), num_seqs,
                           total_tokens, num_heads, sl2);
    } else {
        hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(kThreads), 0, stream, q, k, v, o, qs,
                           ks, vs, os, cu, reinterpret_cast<const int4*>(items), num_seqs,
                           total_tokens, num_heads, sl2);
    }
    return hipGetLastError();
}

}  // namespace h3
