// Padding-free varlen joint attention on bf16 MFMA (gfx950).
//
// Computes, per packed segment and head, O = softmax(Q K^T * scale) V over
// the segment's valid tokens only ("MiniMax H3 FastH3 real-time serving with
// vLLM-Omni", section "System-wide optimizations in vLLM-Omni", long-sequence
// attention bullet; "FastH3 在八卡 B300 上实现完整 MP4 生成快于播放时长",
// section "长序列注意力与通信优化").
//
// Design (CDNA4, 64-lane waves):
//  * one workgroup per work item (head, segment, 256-row query tile), eight
//    waves of 32 query rows, one workgroup per CU (two waves per SIMD); the
//    work list comes from the bookkeeping kernel, so no padded token is ever
//    loaded or computed;
//  * scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane owns one query row (lane % 32) and
//    16 of every 32 keys, so row statistics are lane-local plus one exchange
//    with the lane 32 away; O^T = V^T P^T with P converted to bf16 in
//    registers directly in the MFMA operand layout and V^T fragments read
//    from row-major V through ds_read_b64_tr_b16;
//  * ping-pong: per 64-key tile a wave runs an MFMA block (P V of the
//    previous tile, then S^T of this tile) and a softmax block (exp2, row
//    sums, bf16 P). The two waves of a SIMD run these half a tile apart, one
//    in its MFMA block while the other is in its softmax, with a workgroup
//    barrier at every half tile; both groups run the same instruction
//    stream, the second group shifted by one barrier, which keeps register
//    allocation to a single path (a barrier counts arrivals, not program
//    locations). The softmax VALU work of one wave then hides under the
//    other's MFMAs instead of the two phases alternating on the whole SIMD;
//  * K and V tiles of 64 keys move global -> LDS with buffer_load_dwordx4
//    ... lds from scalar buffer descriptors (rows past the segment end read
//    as zeros, their scores are masked), double buffered, issued by the
//    second group in its softmax half; XOR-swizzled 16-byte chunks keep both
//    fragment reads free of bank conflicts. Fragment reads run a few MFMAs
//    ahead of the MFMA stream;
//  * softmax in the exp2 domain with a reference max that only moves when a
//    lane's partial sum of exp2 values exceeds 2^16 (or is infinite): then
//    the tile's true max is taken, O and l are rescaled and the tile's p
//    recomputed. Between such events p <= 2^16 and O is never touched; the
//    final O / l is the same softmax. Row sums use fp32 adds of the
//    unrounded p.
#include <type_traits>
#include <utility>

#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {
namespace {

constexpr int kBN = 64;        // keys per tile
constexpr int kWaves = 8;      // 32 query rows each; waves w and w + 4 share a SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kRing = 4;       // fragment reads in flight ahead of the MFMA stream

template <int D>
struct Cfg {
    static constexpr int RB = D * 2;
    static constexpr int CPR = D / 8;
    static constexpr int RPI = 1024 / RB;
    static constexpr int NI = kBN / RPI / (kWaves / 2);   // DMA instructions per DMA wave per operand
    static constexpr int TILE = kBN * RB;
    static constexpr int KC = D / 16;
    static constexpr int DB = D / 32;
    static constexpr int NQ = 2 * KC;   // S^T MFMAs per tile
    static constexpr int NP = 4 * DB;   // P V MFMAs per tile
};

template <int D> __device__ __forceinline__ int kswz(int r) { return r % (D / 8); }
template <int D> __device__ __forceinline__ int vswz(int r) {
    return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

constexpr int kBufferWord3 = 0x00020000;

template <class F, int... J>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, J...>) {
    (f(std::integral_constant<int, J>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ void buf_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, void* lds_dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(lds_dst)),
        16, voff, 0, 0, 0);
}

__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) i16x4*>(reinterpret_cast<uintptr_t>(p)));
    return __builtin_bit_cast(u32x2, v);
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, int64_t qs, int64_t ks,
    int64_t vs, int64_t os, const int32_t* __restrict__ cu, const int4* __restrict__ items,
    int num_seqs, int total_tokens, int num_heads, float scale_log2,
    const int32_t* __restrict__ rank_prefix) {
    using C = Cfg<D>;
    constexpr int KC = C::KC, DB = C::DB, RB = C::RB, CPR = C::CPR, NQ = C::NQ, NP = C::NP;
    constexpr int NM = NQ + NP;

    // K stage 0, K stage 1, V stage 0, V stage 1
    __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE];

    const int4 it = items[xcd_item(blockIdx.x, rank_prefix, num_seqs, num_heads)];
    const int head = __builtin_amdgcn_readfirstlane(it.x);
    const int seg = __builtin_amdgcn_readfirstlane(it.y);
    const int q0 = __builtin_amdgcn_readfirstlane(it.z);
    const int qlen = __builtin_amdgcn_readfirstlane(it.w);
    if (seg < 0 || seg >= num_seqs || head < 0 || head >= num_heads) return;
    const int kv0 = max(0, __builtin_amdgcn_readfirstlane(cu[seg]));
    const int kv1 = min(total_tokens, __builtin_amdgcn_readfirstlane(cu[seg + 1]));
    if (q0 < kv0 || qlen <= 0 || q0 + qlen > kv1) return;
    const int len = kv1 - kv0;
    const int ntiles = (len + kBN - 1) / kBN;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;          // 0: MFMA block on even half-tiles, 1: on odd
    const int wg = wave & 3;            // index within the group
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;

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

    // ---- DMA (issued by the group in its softmax half): wave wg of the
    // group fills 1 KB blocks NI*wg .. NI*wg+NI-1 of a tile ----
    const uint16_t* kbase = k + static_cast<int64_t>(head) * D;
    const uint16_t* vbase = v + static_cast<int64_t>(head) * D;
    uint32_t koffb[C::NI], voffb[C::NI];
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
        const int drow = C::RPI * (C::NI * wg + j) + lane / CPR;
        koffb[j] = static_cast<uint32_t>((drow * ks + 8 * ((lane % CPR) ^ kswz<D>(drow))) * 2);
        voffb[j] = static_cast<uint32_t>((drow * vs + 8 * ((lane % CPR) ^ vswz<D>(drow))) * 2);
    }
    auto dma = [&](const uint16_t* base, int64_t stride, const uint32_t (&offb)[C::NI], int tile,
                   char* dst) __attribute__((always_inline)) {
        const int key0 = kv0 + tile * kBN;
        const int rows = min(kBN, kv1 - key0);
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(base + static_cast<int64_t>(key0) * stride), 0,
            static_cast<int>(rows * stride * 2), kBufferWord3);
#pragma unroll
        for (int j = 0; j < C::NI; ++j) buf_dma16(rsrc, offb[j], dst + (C::NI * wg + j) * 1024);
    };
    auto dma_k = [&](int tile) __attribute__((always_inline)) {
        dma(kbase, ks, koffb, tile, smem + (tile & 1) * C::TILE);
    };
    auto dma_v = [&](int tile) __attribute__((always_inline)) {
        dma(vbase, vs, voffb, tile, smem + (2 + (tile & 1)) * C::TILE);
    };

    // ---- LDS fragment offsets ----
    const int ksw = kswz<D>(l32);
    int koff[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) koff[c] = l32 * RB + 16 * ((2 * c + g) ^ ksw);
    const int e4 = (lane & 15) >> 2;
    const int qq = lane & 3;
    const int h16 = (lane >> 4) & 1;
    const int vsw = vswz<D>(4 * g + e4);
    int voff[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        voff[db] = (4 * g + e4) * RB + 16 * ((4 * db + 2 * h16 + (qq >> 1)) ^ vsw) + 8 * (qq & 1);
    auto kfrag = [&](const char* kl, int i) __attribute__((always_inline)) {
        return *reinterpret_cast<const bf16x8*>(kl + 32 * (i & 1) * RB + koff[i >> 1]);
    };
    // P V MFMA i: db = i % DB (consecutive MFMAs on different accumulators),
    // key step (b, t) = ((i / DB) >> 1, (i / DB) & 1)
    auto vfrag = [&](const char* vl, int i) __attribute__((always_inline)) {
        const int db = i % DB, b = (i / DB) >> 1, t = (i / DB) & 1;
        const char* base = vl + (32 * b + 16 * t) * RB + voff[db];
        const u32x2 lo = lds_read_tr16(base);
        const u32x2 hi = lds_read_tr16(base + 8 * RB);
        const u32x4 vf = {lo.x, lo.y, hi.x, hi.y};
        return __builtin_bit_cast(bf16x8, vf);
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) oacc[b] = f32x16{};
    float m_run = -1e30f;
    float l_run = 0.f;
    constexpr float kTrig = 65536.0f;
    f32x16 sc[2];
    bf16x8 pf[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int t = 0; t < 2; ++t) pf[b][t] = bf16x8{};

    // MFMA blocks. Both: O += P(u-1) V(u-1) then S^T = K(u) Q^T, the
    // fragment reads kRing MFMAs ahead across the two; stages are
    // compile-time so LDS offsets are immediates.
    auto qk_pv = [&](auto kst_c) __attribute__((always_inline)) {
        constexpr int kst = decltype(kst_c)::value;       // K(u) stage = u & 1
        const char* kl = smem + kst * C::TILE;
        const char* vl = smem + (2 + (kst ^ 1)) * C::TILE;   // V(u-1)
        auto frag = [&](int j) __attribute__((always_inline)) {
            return j < NQ ? kfrag(kl, j) : vfrag(vl, j - NQ);
        };
        bf16x8 ring[kRing];
        static_for<kRing>([&](auto jc) { ring[decltype(jc)::value] = frag(decltype(jc)::value); });
        static_for<NM>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const bf16x8 a = ring[j % kRing];
            if constexpr (j + kRing < NM) ring[j % kRing] = frag(j + kRing);
            if constexpr (j < NQ) {
                sc[j & 1] = mfma32x32x16(a, qf[j >> 1], j < 2 ? f32x16{} : sc[j & 1]);
            } else {
                constexpr int i = j - NQ;
                oacc[i % DB] = mfma32x32x16(a, pf[(i / DB) >> 1][(i / DB) & 1], oacc[i % DB]);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    auto qk_only = [&]() __attribute__((always_inline)) {      // tile 0, stage 0
        const char* kl = smem;
        bf16x8 ring[kRing];
        static_for<kRing>([&](auto jc) { ring[decltype(jc)::value] = kfrag(kl, decltype(jc)::value); });
        static_for<NQ>([&](auto jc) __attribute__((always_inline)) {
            constexpr int i = decltype(jc)::value;
            const bf16x8 a = ring[i % kRing];
            if constexpr (i + kRing < NQ) ring[i % kRing] = kfrag(kl, i + kRing);
            sc[i & 1] = mfma32x32x16(a, qf[i >> 1], i < 2 ? f32x16{} : sc[i & 1]);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    auto pv_only = [&](int vst) __attribute__((always_inline)) {   // last tile
        const char* vl = smem + (2 + vst) * C::TILE;
#pragma unroll
        for (int i = 0; i < NP; ++i)
            oacc[i % DB] = mfma32x32x16(vfrag(vl, i), pf[(i / DB) >> 1][(i / DB) & 1], oacc[i % DB]);
    };

    // softmax of tile u's scores into P(u): exp2 against the reference max;
    // if a lane's partial sum passes 2^16 (or the first tile), move the
    // reference to the true max, rescale O and l, and redo p
    const int keys_left = len - (ntiles - 1) * kBN;
    auto softmax = [&](int u) __attribute__((always_inline)) {
        if (u + 1 == ntiles && keys_left < kBN) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 32 * b + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (key >= keys_left) sc[b][r] = -INFINITY;
                }
        }
        auto pass = [&](float mb) __attribute__((always_inline)) {
            float ps = 0.f;
#pragma unroll
            for (int r = 0; r < 32; r += 2) {
                const float e0 = __builtin_amdgcn_exp2f(fmaf(sc[r >> 4][r & 15], scale_log2, -mb));
                const float e1 = __builtin_amdgcn_exp2f(fmaf(sc[r >> 4][(r & 15) + 1], scale_log2, -mb));
                ps += e0 + e1;
                const bf16x2 pr = {static_cast<__bf16>(e0), static_cast<__bf16>(e1)};
                pf[r >> 4][(r >> 3) & 1][r & 7] = pr[0];
                pf[r >> 4][(r >> 3) & 1][(r & 7) + 1] = pr[1];
            }
            return ps;
        };
        float psum = pass(m_run * scale_log2);
        if (__any(!(psum <= kTrig))) {
            asm volatile("" ::: "memory");
            float mt = sc[0][0];
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, fmaxf(sc[0][r], sc[1][r]));
            mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
            const float m_new = fmaxf(m_run, mt);
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            psum = pass(m_new * scale_log2);
        }
        l_run += psum;
    };

    // ---- prologue: K(0) in LDS (every wave a share) ----
    {
        const int key0 = kv0;
        const int rows = min(kBN, kv1 - key0);
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(kbase + static_cast<int64_t>(key0) * ks), 0,
            static_cast<int>(rows * ks * 2), kBufferWord3);
        constexpr int NI8 = kBN / C::RPI / kWaves;
#pragma unroll
        for (int j = 0; j < NI8; ++j) {
            const int drow = C::RPI * (NI8 * wave + j) + lane / CPR;
            const uint32_t off = static_cast<uint32_t>((drow * ks + 8 * ((lane % CPR) ^ kswz<D>(drow))) * 2);
            buf_dma16(rsrc, off, smem + (NI8 * wave + j) * 1024);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Every wave runs the same sequence, MFMA block M(u) (P V(u-1), S^T(u))
    // then softmax S(u), with a barrier after each; group 1 runs one
    // half-tile behind group 0 (an extra barrier before its first block, and
    // group 0 an extra one after its last), so in every half-tile one wave of
    // each SIMD issues MFMAs while the other runs its softmax.
    // Group 1 issues the DMA of K(u+2) and V(u+1) at the start of its S(u),
    // i.e. after barrier 2u+2: their stages held K(u) and V(u-1), which M(u)
    // of both groups has read by then. They are next read in M(u+2), from
    // half-tile 2u+4 on; group 1 waits for its DMA at the end of its M(u+1),
    // before barrier 2u+4. (Its V reads in M(u+1) already wait for it: the
    // compiler cannot tell the DMA's LDS stage from the one being read.)
    const bool g0 = grp == 0;
    // LDS writes done and a workgroup barrier; outstanding DMA is waited for
    // only where its data is needed (the memory clobber keeps the compiler
    // from moving LDS accesses across)
    auto bar = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    auto dma_wait = [&]() __attribute__((always_inline)) {
        if (!g0) __builtin_amdgcn_s_waitcnt(0);
    };
    auto issue_dma = [&](int u) __attribute__((always_inline)) {
        if (!g0) {
            if (u + 2 < ntiles) dma_k(u + 2);
            if (u + 1 < ntiles) dma_v(u + 1);
        }
    };
    if (!g0) {
        // K(1), V(0) for M(1)
        if (1 < ntiles) dma_k(1);
        dma_v(0);
        bar();
    }
    qk_only();
    dma_wait();
    bar();
    issue_dma(0);
    softmax(0);
    bar();
    auto tile = [&](int u, auto kst_c) __attribute__((always_inline)) {
        qk_pv(kst_c);
        dma_wait();
        bar();
        issue_dma(u);
        softmax(u);
        bar();
    };
    int u = 1;
    for (; u + 2 <= ntiles; u += 2) {
        tile(u, std::integral_constant<int, 1>{});
        tile(u + 1, std::integral_constant<int, 0>{});
    }
    if (u < ntiles) tile(u, std::integral_constant<int, 1>{});
    pv_only((ntiles - 1) & 1);
    if (g0) bar();

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
                u32x2 w;
                w.x = pack_bf16x2(oacc[db][4 * r4 + 0] * inv, oacc[db][4 * r4 + 1] * inv);
                w.y = pack_bf16x2(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv);
                *reinterpret_cast<u32x2*>(op + d) = w;
            }
    }
}

}  // namespace

hipError_t launch_attn_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            uint16_t* o, int64_t qs, int64_t ks, int64_t vs, int64_t os,
                            const int32_t* cu, const int32_t* items, int64_t num_items,
                            int num_seqs, int total_tokens, int num_heads, int head_dim,
                            float softmax_scale, const int32_t* rank_prefix, hipStream_t stream) {
    if (num_items <= 0) return hipSuccess;
    const float sl2 = softmax_scale * kLog2e;
    const dim3 grid(static_cast<unsigned>(num_items));
    if (head_dim == 128) {
        hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(kThreads), 0, stream, q, k, v, o, qs,
                           ks, vs, os, cu, reinterpret_cast<const int4*>(items), num_seqs,
                           total_tokens, num_heads, sl2, rank_prefix);
    } else {
        hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(kThreads), 0, stream, q, k, v, o, qs,
                           ks, vs, os, cu, reinterpret_cast<const int4*>(items), num_seqs,
                           total_tokens, num_heads, sl2, rank_prefix);
    }
    return hipGetLastError();
}

}  // namespace h3
