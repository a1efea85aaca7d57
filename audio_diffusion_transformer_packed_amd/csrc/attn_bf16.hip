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
//    waves of 32 query rows each, one workgroup per CU (two waves per SIMD);
//    the 256 rows share every K / V tile brought into LDS, which halves the
//    global -> LDS traffic of a 128-row tile; the work list comes from the
//    bookkeeping kernel, so no padded token is ever loaded or computed;
//  * scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane owns one query row (lane % 32) and
//    16 of every 32 keys, so row statistics are lane-local plus one exchange
//    with the lane 32 away;
//  * O^T = V^T P^T: P stays in registers, converted to bf16 directly in the
//    MFMA operand layout; V^T fragments come from row-major V in LDS through
//    ds_read_b64_tr_b16 (transposing 16-lane read);
//  * K and V tiles of 64 keys move global -> LDS with buffer_load_dwordx4
//    ... lds (no staging registers; the tile base lives in scalar registers,
//    so the DMA costs no vector address arithmetic), double buffered, with
//    XOR-swizzled 16-byte chunks so both fragment reads are free of bank
//    conflicts;
//  * each key tile: S^T MFMAs, softmax, P V MFMAs, while the next tile's K
//    and V stream into the other LDS stage; the two waves of a SIMD overlap
//    one wave's softmax with the other's MFMAs;
//  * softmax in the exp2 domain with a reference max that only moves when a
//    lane's partial sum of exp2 values exceeds 2^16 (or is infinite):
//    then the tile's true max is taken, O and l are rescaled and the tile's
//    p recomputed. Between such events p <= 2^16 and O is never touched; the
//    final O / l is the same softmax. Row sums use fp32 adds, not v_dot2,
//    which would occupy the matrix pipe.
#include <type_traits>

#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {
namespace {

constexpr int kBN = 64;        // keys per tile
constexpr int kWaves = 8;      // 32 query rows each
constexpr int kThreads = 64 * kWaves;

template <int D>
struct Cfg {
    static constexpr int RB = D * 2;               // bytes per K / V row in LDS
    static constexpr int CPR = D / 8;              // 16-byte chunks per row
    static constexpr int RPI = 1024 / RB;          // rows per 1 KB DMA instruction
    static constexpr int NI = kBN / RPI / kWaves;       // DMA instructions per wave per operand
    static constexpr int TILE = kBN * RB;          // bytes per K or V tile
    static constexpr int KC = D / 16;              // MFMA k-steps over the head dim
    static constexpr int DB = D / 32;              // 32-wide output blocks
};

// Chunk swizzles (physical chunk = logical chunk ^ swizzle(row)).
// K: fragment reads take one chunk of 32 consecutive rows; row % CPR spreads them.
// V: a transposing read takes 4 chunks (64 B) of 8 consecutive rows; the
// swizzle moves neighbouring rows to different 64-byte quarters.
template <int D> __device__ __forceinline__ int kswz(int r) { return r % (D / 8); }
template <int D> __device__ __forceinline__ int vswz(int r) {
    return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// Buffer resource word 3 for raw (untyped, stride 0) access on gfx9-family
// parts: 32-bit data format; out-of-range loads return zero.
constexpr int kBufferWord3 = 0x00020000;

// 16 bytes per lane from buffer offset `voff` straight into LDS at lds_dst
// (lane i writes lds_dst + 16 i), no staging registers.
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
    int num_seqs, int total_tokens, int num_heads, float scale_log2) {
    using C = Cfg<D>;
    constexpr int KC = C::KC, DB = C::DB, RB = C::RB, CPR = C::CPR;

    // K stage 0, K stage 1, V stage 0, V stage 1
    __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE];

    // work-item fields and segment bounds are workgroup-uniform: keep them in
    // scalar registers (so the K / V buffer descriptors are scalar too)
    const int4 it = items[blockIdx.x];
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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
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

    // ---- DMA: instruction i of a tile fills rows RPI*i .. RPI*i+RPI-1;
    // this wave issues i = NI*wave + j; lane -> row RPI*i + lane/CPR, physical
    // chunk lane % CPR, which holds logical chunk (lane % CPR) ^ swizzle(row).
    // A buffer resource based at the tile's first row (scalar registers) and
    // sized to the segment's remaining rows makes every tile one code path:
    // rows past the segment end are out of range and load as zeros, and
    // their scores are masked to -inf in the last tile.
    const uint16_t* kbase = k + static_cast<int64_t>(head) * D;
    const uint16_t* vbase = v + static_cast<int64_t>(head) * D;
    uint32_t koffb[C::NI], voffb[C::NI];      // byte offsets from the tile's first row
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
        const int drow = C::RPI * (C::NI * wave + j) + lane / CPR;
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
        for (int j = 0; j < C::NI; ++j) buf_dma16(rsrc, offb[j], dst + (C::NI * wave + j) * 1024);
    };
    auto dma_k = [&](int tile, int stage) __attribute__((always_inline)) {
        dma(kbase, ks, koffb, tile, smem + stage * C::TILE);
    };
    auto dma_v = [&](int tile, int stage) __attribute__((always_inline)) {
        dma(vbase, vs, voffb, tile, smem + (2 + stage) * C::TILE);
    };

    // ---- LDS read offsets ----
    // K fragment (A operand of S^T): rows 32b + l32, logical chunk 2c + g.
    const int ksw = kswz<D>(l32);
    int koff[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) koff[c] = l32 * RB + 16 * ((2 * c + g) ^ ksw);
    // V^T fragment by transposing read: in each 16-lane group, lane 4e + qq
    // addresses V[row0 + e][dbase + 4 qq] with row0 = 32b + 16t + 8 half + 4g
    // and dbase = 32 db + 16 h16; lane j of the group then receives
    // V[row0 + e][dbase + j] for e = 0..3.
    const int e4 = (lane & 15) >> 2;
    const int qq = lane & 3;
    const int h16 = (lane >> 4) & 1;
    const int vsw = vswz<D>(4 * g + e4);
    int voff[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        voff[db] = (4 * g + e4) * RB + 16 * ((4 * db + 2 * h16 + (qq >> 1)) ^ vsw) + 8 * (qq & 1);

    f32x16 oacc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) oacc[b] = f32x16{};
    // reference max (raw score units) of this lane's row; a large finite start
    // value makes the first tile trigger through an infinite sum, never NaN
    float m_run = -1e30f;
    float l_run = 0.f;         // partial row sum over this lane's keys
    constexpr float kTrig = 65536.0f;

    // S^T(tile) from K stage `stage`; K fragments are read PK MFMAs ahead
    auto qk = [&](int stage, f32x16 (&sc)[2]) __attribute__((always_inline)) {
        const char* kl = smem + stage * C::TILE;
        constexpr int NM = 2 * KC, PK = 3;
        auto kfrag = [&](int i) __attribute__((always_inline)) {
            return *reinterpret_cast<const bf16x8*>(kl + 32 * (i & 1) * RB + koff[i >> 1]);
        };
        sc[0] = f32x16{};
        sc[1] = f32x16{};
        bf16x8 kq[PK];
#pragma unroll
        for (int i = 0; i < PK; ++i) kq[i] = kfrag(i);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            bf16x8 kn;
            if (i + PK < NM) kn = kfrag(i + PK);
            sc[i & 1] = mfma32x32x16(kq[i % PK], qf[i >> 1], sc[i & 1]);
            __builtin_amdgcn_sched_barrier(0);
            if (i + PK < NM) kq[i % PK] = kn;
        }
    };

    // exp2 of score r of a tile against the current reference max
    auto pexp = [&](const f32x16 (&s)[2], int r, float mb) __attribute__((always_inline)) {
        return __builtin_amdgcn_exp2f(fmaf(s[r >> 4][r & 15], scale_log2, -mb));
    };
    // bf16 P in the B-operand layout: pf[b][t][e] = p of score 16 b + 8 t + e.
    // The row sum adds the fp32 p with plain adds: v_dot2 (a dot on the
    // rounded pair) would share the matrix pipe and stall the other wave's
    // MFMAs, and the bf16 rounding of P is unbiased, so l of the unrounded p
    // normalises the same softmax to well inside the bf16 error.
    auto put = [&](bf16x8 (&pf)[2][2], int r, float v0, float v1, float& sum) __attribute__((always_inline)) {
        const bf16x2 pr = {static_cast<__bf16>(v0), static_cast<__bf16>(v1)};
        pf[r >> 4][(r >> 3) & 1][r & 7] = pr[0];
        pf[r >> 4][(r >> 3) & 1][(r & 7) + 1] = pr[1];
        sum += v0 + v1;
    };

    // plain exp / sum / bf16 of one tile's scores
    auto softmax_exp = [&](const f32x16 (&s)[2], bf16x8 (&pf)[2][2], float& psum) __attribute__((always_inline)) {
        const float mb = m_run * scale_log2;
        psum = 0.f;
#pragma unroll
        for (int r = 0; r < 32; r += 2) {
            put(pf, r, pexp(s, r, mb), pexp(s, r + 1, mb), psum);
        }
    };

    // If any lane's sum exceeded 2^16 (a new max far above the reference, or
    // the first tile), move the reference to the true max, rescale O and l,
    // and redo the tile's p. Then accumulate l.
    auto softmax_fix = [&](const f32x16 (&s)[2], bf16x8 (&pf)[2][2], float psum) __attribute__((always_inline)) {
        if (__any(!(psum <= kTrig))) {            // wave-uniform
            asm volatile("" ::: "memory");
            float mt = s[0][0];
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, fmaxf(s[0][r], s[1][r]));
            mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
            const float m_new = fmaxf(m_run, mt);
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            softmax_exp(s, pf, psum);
        }
        l_run += psum;
    };

    // O^T += V^T P^T from V stage `stage`; k-step (b, t) covers keys
    // 32b + 16t + [0, 16): lane half g holds keys 4g + [0,4) and 8 + 4g + [0,4)
    // of it (the S^T accumulator rows), the transposing reads fetch the same.
    auto pv = [&](int stage, const bf16x8 (&pf)[2][2]) __attribute__((always_inline)) {
        const char* vl = smem + (2 + stage) * C::TILE;
        // MFMA i: db = i / 4, (b, t) = (i / 2 % 2, i % 2); fragments read ahead
        auto frag = [&](int i) __attribute__((always_inline)) {
            const int db = i >> 2, b = (i >> 1) & 1, t = i & 1;
            const char* base = vl + (32 * b + 16 * t) * RB + voff[db];
            const u32x2 lo = lds_read_tr16(base);
            const u32x2 hi = lds_read_tr16(base + 8 * RB);
            const u32x4 vf = {lo.x, lo.y, hi.x, hi.y};
            return __builtin_bit_cast(bf16x8, vf);
        };
        constexpr int NM = 4 * DB, PV_AHEAD = 2;
        bf16x8 vq[PV_AHEAD];
#pragma unroll
        for (int i = 0; i < PV_AHEAD; ++i) vq[i] = frag(i);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            bf16x8 vn;
            if (i + PV_AHEAD < NM) vn = frag(i + PV_AHEAD);
            oacc[i >> 2] = mfma32x32x16(vq[i % PV_AHEAD], pf[(i >> 1) & 1][i & 1], oacc[i >> 2]);
            __builtin_amdgcn_sched_barrier(0);
            if (i + PV_AHEAD < NM) vq[i % PV_AHEAD] = vn;
        }
    };

    auto mask_tail = [&](f32x16 (&s)[2], int keys_left) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 32 * b + 8 * (r >> 2) + 4 * g + (r & 3);
                if (key >= keys_left) s[b][r] = -INFINITY;
            }
    };

    f32x16 sc[2];
    bf16x8 pf[2][2];
    float psum;

    // Tile t sits in K / V stage t % 2. Iteration t: DMA tile t+1 into the
    // other stage, then S^T(t), softmax(t), P V(t) from this stage, then wait
    // for the DMA and a barrier (one per tile). The loop runs two tiles per
    // trip so each stage is a compile-time constant and the LDS stage offsets
    // fold into the fragment reads' immediate offsets.
    dma_k(0, 0);
    dma_v(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int keys_left = len - (ntiles - 1) * kBN;
    auto tile = [&](int t, auto stage_c) __attribute__((always_inline)) {
        constexpr int stage = decltype(stage_c)::value;
        const bool last = t + 1 == ntiles;
        if (!last) {
            dma_k(t + 1, stage ^ 1);
            dma_v(t + 1, stage ^ 1);
        }
        qk(stage, sc);
        if (last && keys_left < kBN) mask_tail(sc, keys_left);
        softmax_exp(sc, pf, psum);
        softmax_fix(sc, pf, psum);
        pv(stage, pf);
        if (!last) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    };
    for (int t = 0; t < ntiles; t += 2) {
        tile(t, std::integral_constant<int, 0>{});
        if (t + 1 < ntiles) tile(t + 1, std::integral_constant<int, 1>{});
    }

    // ---- normalise and store: lane holds dims 32 db + 8 r4 + 4 g + [0, 4) ----
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
