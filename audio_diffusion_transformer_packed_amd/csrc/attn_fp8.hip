// fp8 (e4m3) varlen attention with skip-softmax on gfx950 fp8 MFMA
// ("MiniMax H3 FastH3 real-time serving with vLLM-Omni", section "Scaling
// beyond the FastH3 profile", sparse & quantized attention bullet; "FastH3
// 在八卡 B300 上实现完整 MP4 生成快于播放时长", section "其他加速路径：有损但可控":
// SAGE quantises attention to FP8, Skip-Softmax skips the Softmax and P x V
// work of unimportant parts while Q K^T is still computed).
//
// Per segment and head, over the codes and scales written by the quantise
// pass (fp8_quant.hip):
//   S = (Q8 K8^T) s_q s_k * scale, online softmax over 64-key tiles in
//   ascending order with the exact running row max m,
//   P8 = e4m3(448 p), p = exp(S - m), l = the row sum of P8 (one
//   16x16x128 MFMA per tile against a 0/1 operand, in place of 32 fp32
//   adds),
//   O = (sum P8 V8) s_v / (448 l).
// Skip rule: for the 32 query rows of a wave, a key tile other than the
// segment's first is skipped (no exp, no P V contribution) when every
// valid row has its tile maximum more than `threshold` (natural-log units)
// below its running maximum. Each work item reports its number of skipped (32-row group, key
// tile) pairs; the count is summed in LDS, no atomics.
//
// Design (CDNA4): the bf16 kernel's layout with v_mfma_f32_32x32x64_f8f6f4.
//  * one workgroup of eight waves per 256-row work item, 32 query rows per
//    wave, each lane owning one query row of S^T = K Q^T (lane % 32);
//  * K tiles (64 keys x 128 B) and V^T tiles (128 channels x 64 B, keys
//    already in the lanes' P order) are contiguous 8 KB blocks in HBM, moved
//    to LDS with buffer_load_dwordx4 ... lds through scalar descriptors (no
//    vector address arithmetic), double buffered, XOR-swizzled for
//    conflict-free 16-byte fragment reads; no transposing reads are needed;
//  * P is converted to e4m3 in registers, already in the B-operand byte
//    order of the P V MFMA; per tile a wave issues 4 + 4 fp8 MFMAs;
//  * ping-pong: the two waves of a SIMD run their MFMA and softmax blocks
//    half a tile apart (see the bf16 kernel), so one wave's softmax VALU
//    work overlaps the other's MFMAs.
//
// The same kernel, instantiated with BSA = true, runs the block-sparse
// attention ("MiniMax H3 on Ascend 950PR / 950DT", section "Recommended
// lossy configuration (Ascend 950PR / 950DT)": EQBSA, Q/K in INT8 and V in
// FP8): Q and K hold INT8 codes (fp8_quant.hip's INT8 variant), S^T runs on
// v_mfma_i32_32x32x32_i8 accumulating onto the bits of 1.5 * 2^23 (read as
// fp32 that is the score plus an exact offset, folded into the exp2
// argument's constant: no int-to-float converts), and each work item walks
// only its query block's kept key tiles (bsa_select.hip), staged with their
// K scales in LDS before the loop; V, P and the softmax are the fp8 path's.
#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {
namespace {

constexpr int kD = 128;
constexpr int kBN = 64;                    // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKT = kBN * kD;              // bytes of a K tile
constexpr int kVT = kD * kBN;              // bytes of a V^T tile
constexpr float kLog2_448 = 8.807354922057604f;
constexpr float kBsaMagic = 12582912.0f;   // 1.5 * 2^23, the BSA score offset

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_fp8_16(i32x8 a, i32x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Buffer resource word 3 for raw (untyped, stride 0) access on gfx9-family
// parts: 32-bit data format; out-of-range loads return zero.
constexpr int kBufferWord3 = 0x00020000;

// 16 bytes per lane from buffer offset voff + soff straight into LDS at
// lds_dst (lane i writes lds_dst + 16 i), no staging registers.
__device__ __forceinline__ void buf_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, int soff,
                                          void* lds_dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(lds_dst)),
        16, voff, soff, 0, 0);
}

// Chunk swizzles (physical 16-byte chunk = logical chunk ^ swizzle(row)):
// K rows are 128 B (8 chunks), V^T rows 64 B (4 chunks).
__device__ __forceinline__ int kswz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int vswz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ i32x8 read32(const char* p0, const char* p1) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p0);
    const u32x4 b = *reinterpret_cast<const u32x4*>(p1);
    return i32x8{static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z), static_cast<int>(a.w),
                 static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z), static_cast<int>(b.w)};
}

__device__ __forceinline__ i32x16 mfma_i8(i32x4 a, i32x4 b, i32x16 c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// BSA: the block-sparse variant. Q and K hold INT8 codes and S^T runs on
// v_mfma_i32_32x32x32_i8 (two per fp8 k-step: the lane's first and second
// 16 bytes; the A and B lanes hold the same head-dim positions, so the sum
// covers every position once); the work item visits only the kept key
// blocks of its query block, lists[(head, first 64-row block)][0 .. keep),
// in ascending order; no skip rule.
// SKIP: the skip rule is compiled in (dense path only); a skipped tile
// saves its exp, convert and rescale (a wave-uniform branch) and leaves P
// zero, so the P V MFMAs, still issued, add nothing.
template <bool BSA, bool SKIP>
__global__ __launch_bounds__(kThreads, 1) void attn_fp8_kernel(
    const uint8_t* __restrict__ q8, const uint8_t* __restrict__ k8, const uint8_t* __restrict__ v8t,
    const float* __restrict__ qsc, const float* __restrict__ ksc, const float* __restrict__ vsc,
    uint16_t* __restrict__ o, int64_t os, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ tb, const int4* __restrict__ items, int num_seqs,
    int total_tokens, int num_heads, int64_t num_tiles, float scale_log2,
    float thr_log2, int32_t* __restrict__ skip_counts, const int32_t* __restrict__ lists,
    int64_t list_stride, int sp_permille, const int32_t* __restrict__ rank_prefix) {
    // K stage 0, K stage 1, V stage 0, V stage 1
    __shared__ __attribute__((aligned(1024))) char smem[2 * kKT + 2 * kVT];
    __shared__ int32_t wskip[kWaves];
    // BSA: kept tiles and their K scales, staged once (no dependent global
    // loads inside the tile loop)
    __shared__ int32_t s_tile[BSA ? kBsaMaxKeyBlocks : 1];
    __shared__ float s_sk[BSA ? kBsaMaxKeyBlocks : 1];

    const int tid = threadIdx.x;
    // work-item fields and segment bounds are workgroup-uniform: keep them in
    // scalar registers (so the tile buffer descriptors are scalar too)
    // Work items go to the XCDs by head (xcd_item, as in the bf16 kernel):
    // the items an XCD runs at one time are neighbouring query blocks of one
    // head, whose K/V (and, block-sparse, whose overlapping kept key blocks)
    // stream through its L2 together. Where that mapping does not apply (head
    // count not a multiple of 8) the block-sparse pass deals chunks of 16
    // consecutive items instead, XCD x taking chunks x, x + 8, ... (ids past
    // the last whole round of 8 x 16 map to themselves). At 57,960 tokens x
    // 24 heads the chunks were 3.7 % faster than list order on frame-local
    // input (0.9 % on i.i.d.), the per-head mapping 1.3 % faster again.
    unsigned item = static_cast<unsigned>(xcd_item(blockIdx.x, rank_prefix, num_seqs, num_heads));
    if (BSA && (rank_prefix == nullptr || (num_heads & 7) != 0)) {
        constexpr unsigned kChunk = 16;
        const unsigned full = gridDim.x / (8 * kChunk) * (8 * kChunk);
        if (blockIdx.x < full) {
            const unsigned x = blockIdx.x % 8, k = blockIdx.x / 8;
            item = (8 * (k / kChunk) + x) * kChunk + k % kChunk;
        }
    }
    const int4 it = items[item];
    const int head = __builtin_amdgcn_readfirstlane(it.x);
    const int seg = __builtin_amdgcn_readfirstlane(it.y);
    const int q0 = __builtin_amdgcn_readfirstlane(it.z);
    const int qlen = __builtin_amdgcn_readfirstlane(it.w);
    bool ok = seg >= 0 && seg < num_seqs && head >= 0 && head < num_heads;
    const int kv0 = ok ? max(0, __builtin_amdgcn_readfirstlane(cu[seg])) : 0;
    const int kv1 = ok ? min(total_tokens, __builtin_amdgcn_readfirstlane(cu[seg + 1])) : 0;
    ok = ok && q0 >= kv0 && qlen > 0 && q0 + qlen <= kv1;
    if (!ok) {
        if (skip_counts && tid == 0) skip_counts[item] = 0;
        return;
    }
    const int len = kv1 - kv0;
    const int ntiles = (len + kBN - 1) / kBN;
    const int keys_left = len - (ntiles - 1) * kBN;
    const int tbs = __builtin_amdgcn_readfirstlane(tb[seg]);
    int nsel = ntiles;                  // key tiles this work item visits
    if constexpr (BSA) {
        nsel = max(1, ntiles - static_cast<int>((static_cast<int64_t>(ntiles) * sp_permille) / 1000));
        nsel = min(nsel, kBsaMaxKeyBlocks);
        const int32_t* lst = lists + (static_cast<int64_t>(head) * num_tiles + tbs + (q0 - kv0) / kBN) * list_stride;
        // clamped into the segment, so no list content can address outside it
        for (int i = tid; i < nsel; i += kThreads) {
            const int t = min(max(lst[i], 0), ntiles - 1);
            s_tile[i] = t;
            s_sk[i] = ksc[static_cast<int64_t>(tbs + t) * num_heads + head];
        }
        __syncthreads();
    }
    // key tile of step u: the u-th kept block, or tile u
    auto tile_at = [&](int u) __attribute__((always_inline)) -> int {
        if constexpr (BSA) return __builtin_amdgcn_readfirstlane(s_tile[u]);
        else return u;
    };

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int qrow_local = wave * 32 + l32;
    const bool qvalid = qrow_local < qlen;
    const bool wave_active = wave * 32 < qlen;   // wave-uniform
    const int64_t row_bytes = static_cast<int64_t>(num_heads) * kD;

    // Q fragments (B operand of S^T): k-step c holds bytes 64c + 32g + [0, 32)
    i32x8 qf[2];
    {
        const uint8_t* qp = q8 + static_cast<int64_t>(q0 + qrow_local) * row_bytes + head * kD + 32 * g;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            if (qvalid) {
                qf[c] = read32(reinterpret_cast<const char*>(qp + 64 * c),
                               reinterpret_cast<const char*>(qp + 64 * c + 16));
            } else {
                qf[c] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
            }
        }
    }
    // s_q * scale * log2(e) of this lane's row
    const int qblk = tbs + (q0 - kv0 + min(qrow_local, qlen - 1)) / kBN;
    const float sq = qsc[static_cast<int64_t>(qblk) * num_heads + head] * scale_log2;

    // Ping-pong as in the bf16 kernel: waves 0-3 and 4-7 (the two waves of
    // each SIMD) run the same sequence of MFMA blocks M(u) (S^T of tile u,
    // P V of tile u-1) and softmax blocks S(u), half a tile apart, with a
    // workgroup barrier between consecutive blocks; the second group issues
    // the DMA at the start of its softmax block.
    const int grp = wave >> 2;
    const bool g0 = grp == 0;
    const int wg = wave & 3;
    // DMA: 1 KB block j of a tile: K rows 8 j + lane / 8 (chunk lane % 8),
    // V^T rows 16 j + lane / 4 (chunk lane % 4), each loading the logical
    // chunk that the swizzle puts there. The second group's wave wg fills
    // blocks 2 wg and 2 wg + 1; in the prologue every wave fills K block `wave`.
    auto ksrc_of = [&](int j) __attribute__((always_inline)) {
        const int krow = 8 * j + (lane >> 3);
        return static_cast<uint32_t>(krow * kD + 16 * ((lane & 7) ^ kswz(krow)));
    };
    auto vsrc_of = [&](int j) __attribute__((always_inline)) {
        const int vrow = 16 * j + (lane >> 2);
        return static_cast<uint32_t>(vrow * kBN + 16 * ((lane & 3) ^ vswz(vrow)));
    };
    const uint32_t ksrc0 = ksrc_of(2 * wg), ksrc1 = ksrc_of(2 * wg + 1);
    const uint32_t vsrc0 = vsrc_of(2 * wg), vsrc1 = vsrc_of(2 * wg + 1);
    // one descriptor per operand covering this segment's tiles of this head;
    // the tile is the scalar offset of each load
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(k8 + (static_cast<int64_t>(head) * num_tiles + tbs) * kKT), 0,
        ntiles * kKT, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(v8t + (static_cast<int64_t>(head) * num_tiles + tbs) * kVT), 0,
        ntiles * kVT, kBufferWord3);
    // step u's tiles go to stage u & 1, passed as a compile-time parity
    // (par_c, an integral_constant) so that stage offsets are immediates
    auto dma_k = [&](int u, auto par_c) __attribute__((always_inline)) {
        constexpr int par = decltype(par_c)::value;
        char* dst = smem + par * kKT + 2048 * wg;
        const int tile = tile_at(u);
        buf_dma16(rk, ksrc0, tile * kKT, dst);
        buf_dma16(rk, ksrc1, tile * kKT, dst + 1024);
    };
    auto dma_v = [&](int u, auto par_c) __attribute__((always_inline)) {
        constexpr int par = decltype(par_c)::value;
        char* dst = smem + 2 * kKT + par * kVT + 2048 * wg;
        const int tile = tile_at(u);
        buf_dma16(rv, vsrc0, tile * kVT, dst);
        buf_dma16(rv, vsrc1, tile * kVT, dst + 1024);
    };

    // LDS fragment offsets. K block b, k-step c: row 32b + l32, logical
    // chunks 4c + 2g + {0, 1}. V^T block db: row 32db + l32, chunks 2g + {0, 1}.
    const int ksw = kswz(l32), vsw = vswz(l32);
    int kro[2][2], vro[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) kro[c][h] = l32 * kD + 16 * ((4 * c + 2 * g + h) ^ ksw);
#pragma unroll
    for (int h = 0; h < 2; ++h) vro[h] = l32 * kBN + 16 * ((2 * g + h) ^ vsw);

    f32x16 oacc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) oacc[b] = f32x16{};
    float m_run = -1e30f;     // running row max, exp2 units (finite start: no inf - inf)
    // row sums of P8 = e4m3(448 p): one v_mfma_f32_16x16x128_f8f6f4 per
    // tile with P (as held for the P V MFMA) as its B operand. Read that way
    // lane l supplies query l % 32 as column l % 16 of k-group l / 16, so an
    // A operand of e4m3 ones (0x38) where the k-group's parity equals the
    // row's parity, zeros elsewhere, makes even output rows the sums of query
    // l % 16 and odd rows those of query l % 16 + 16: lacc[0] and lacc[1]
    // (read and rescaled; [2] and [3] repeat them). Half the matrix-core
    // cycles of a 32x32x64 MFMA against an all-ones operand.
    f32x4 lacc = f32x4{0.f, 0.f, 0.f, 0.f};
    const int pat = ((lane >> 4) & 1) == (lane & 1) ? 0x38383838 : 0;
    i32x8 ones = {pat, pat, pat, pat, pat, pat, pat, pat};
    // opaque from here on: kept in its eight registers through the tile loop
    // (as a known value the compiler rebuilt it from one register with
    // seven moves per tile)
    asm volatile("" : "+v"(ones));
    // BSA: the INT8 score accumulators start from this block (the bits of
    // 1.5 * 2^23 in every element), opaque for the same reason (set per
    // tile it cost eight 64-bit moves)
    i32x16 magic;
    if constexpr (BSA) {
#pragma unroll
        for (int r = 0; r < 16; ++r) magic[r] = 0x4B400000;
        asm volatile("" : "+v"(magic));
    }
    // SKIP: this wave's skipped-tile count, kept in a vector register (a
    // scalar counter adds to the kernel's scalar register pressure, which
    // then spills inside the tile loop); the empty asm defines it per lane
    int nskip;
    asm volatile("v_mov_b32 %0, 0" : "=v"(nskip));
    // per lane: padding rows never keep a tile (their cut is +inf)
    const float thr_eff = qvalid ? thr_log2 : -INFINITY;
    f32x16 sc[2] = {f32x16{}, f32x16{}};
    i32x8 pf = i32x8{0, 0, 0, 0, 0, 0, 0, 0};

    // MFMA block M(u): S^T(u) from K stage u & 1 (u < T), O += P(u-1) V(u-1)
    // from V stage (u-1) & 1 (u >= 1). A tile the skip rule drops leaves P
    // zero, so its P V adds nothing: the block has no branch around the P V
    // MFMAs (such a branch cost 3-4 % of the kernel when nothing is skipped,
    // more than the MFMAs it saves when tiles are).
    auto mfma_qk = [&](int u, auto par_c) __attribute__((always_inline)) {
        constexpr int par = decltype(par_c)::value;   // u & 1
        if (u < nsel) {
            const char* kl = smem + par * kKT;
            if constexpr (BSA) {
                // accumulate onto the bits of 1.5 * 2^23 (`magic`, the first
                // MFMA's accumulator input): |S| <= 127 * 127 * 128 < 2^22, so
                // each result, read as fp32, is exactly 1.5 * 2^23 + S (no convert)
                i32x16 si[2];
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        const i32x8 kf = read32(kl + 4096 * b + kro[c][0], kl + 4096 * b + kro[c][1]);
                        si[b] = mfma_i8(kf.lo, qf[c].lo, c == 0 ? magic : si[b]);
                        si[b] = mfma_i8(kf.hi, qf[c].hi, si[b]);
                    }
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sc[b][r] = __int_as_float(si[b][r]);
            } else {
                sc[0] = f32x16{};
                sc[1] = f32x16{};
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int b = 0; b < 2; ++b)
                        sc[b] = mfma_fp8(read32(kl + 4096 * b + kro[c][0], kl + 4096 * b + kro[c][1]), qf[c], sc[b]);
            }
        }
    };
    auto mfma_pv = [&](auto par_c) __attribute__((always_inline)) {
        constexpr int par = decltype(par_c)::value;   // u & 1; V(u-1) is in stage 1 - par
        const char* vl = smem + 2 * kKT + (1 - par) * kVT;
#pragma unroll
        for (int db = 0; db < 4; ++db)
            oacc[db] = mfma_fp8(read32(vl + 2048 * db + vro[0], vl + 2048 * db + vro[1]), pf, oacc[db]);
        lacc = mfma_fp8_16(ones, pf, lacc);
    };
    auto mfma_block = [&](int u, auto par_c) __attribute__((always_inline)) {
        if (!wave_active) return;
        mfma_qk(u, par_c);
        if (u >= 1) mfma_pv(par_c);
    };
    // softmax block S(u): tile max, skip rule, rescale, P of tile u
    auto softmax_block = [&](int u) __attribute__((always_inline)) {
        if (!wave_active) return;
        const int tile = tile_at(u);
        float sk;
        if constexpr (BSA) sk = s_sk[u];
        else sk = ksc[static_cast<int64_t>(tbs + u) * num_heads + head];
        if (tile + 1 == ntiles && keys_left < kBN) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * b + 8 * (r >> 2) + 4 * g + (r & 3) >= keys_left) sc[b][r] = -INFINITY;
        }
        // the tile max as a chain of NaN-propagating maxima (v_maximum3_f32,
        // two scores per instruction): scores are finite or -inf, and fmaxf
        // here made the compiler quiet every MFMA result first (one more
        // instruction per score)
        float mx = sc[0][0];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, sc[0][r]), sc[1][r]);
        // lanes l and l ^ 32 hold the same row: one v_permlane32_swap leaves
        // the pair's two values in the two outputs (in either order), with no
        // LDS round trip on the way to the exponentials
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        const float ct = sq * sk;          // exp2 units per raw score
        // BSA scores carry the 1.5 * 2^23 offset (exact to remove from the max)
        const float tmax = (BSA ? mx - kBsaMagic : mx) * ct;
        float m_new = __builtin_elementwise_maximum(m_run, tmax);
        bool run_tile = true;
        if constexpr (SKIP) {
            if (u > 0) {
                if (__builtin_expect(__all(tmax < m_run - thr_eff), 0)) {   // wave-uniform
                    run_tile = false;
                    ++nskip;
                    m_new = m_run;                    // a skipped tile moves no maximum
                }
            }
        }
        if (__any(m_new > m_run)) {                   // wave-uniform
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            // lacc[0] / lacc[1] of lane l hold queries l % 16 and l % 16 + 16,
            // whose factors sit in lanes l & ~16 and l | 16: one
            // v_permlane16_swap of alpha with itself yields both (no LDS)
            const auto af = __builtin_amdgcn_permlane16_swap(__float_as_uint(alpha), __float_as_uint(alpha), false, false);
            lacc[0] *= __uint_as_float(af[0]);
            lacc[1] *= __uint_as_float(af[1]);
#pragma unroll
            for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
        }
        m_run = m_new;
        if (__builtin_expect(run_tile, 1)) {
            // 448 p = exp2(s ct - m + log2 448); bytes in B-operand order:
            // byte 16 b + r of this lane holds score sc[b][r]
            // BSA: the offset's share, 1.5 * 2^23 ct, moves into the constant
            // (one fp32 rounding of that product, below an ulp of it)
            const float mb = BSA ? fmaf(kBsaMagic, ct, m_new - kLog2_448) : m_new - kLog2_448;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const int b = w >> 2, r = 4 * (w & 3);
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[b][r], ct, -mb));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[b][r + 1], ct, -mb));
                const float p2 = __builtin_amdgcn_exp2f(fmaf(sc[b][r + 2], ct, -mb));
                const float p3 = __builtin_amdgcn_exp2f(fmaf(sc[b][r + 3], ct, -mb));
                // the second convert overwrites the upper half: the word's
                // previous value as the first one's "old" saves zeroing it
                int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pf[w], false);
                word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
                pf[w] = word;
            }
        }
        if constexpr (SKIP) {
            if (!run_tile) pf = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    };

    // ---- prologue: K(0) in LDS, every wave one 1 KB block ----
    buf_dma16(rk, ksrc_of(wave), tile_at(0) * kKT, smem + 1024 * wave);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // LDS reads done (so the next DMA may overwrite), workgroup barrier; the
    // memory clobber keeps the compiler from moving LDS accesses across
    auto bar = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    auto dma_wait = [&]() __attribute__((always_inline)) {
        if (!g0) __builtin_amdgcn_s_waitcnt(0);
    };
    // The second group issues K(u+2), V(u+1) at the start of its S(u), after
    // barrier 2u+2: their stages held K(u), V(u-1), which M(u) of both
    // groups has read. They are next read in M(u+2), from half-tile 2u+4 on;
    // the group waits for its DMA at the end of its M(u+1), before barrier 2u+4.
    using Even = std::integral_constant<int, 0>;
    using Odd = std::integral_constant<int, 1>;
    auto issue_dma = [&](int u, auto par_c) __attribute__((always_inline)) {
        constexpr int par = decltype(par_c)::value;
        if (!g0) {
            if (u + 2 < nsel) dma_k(u + 2, par_c);
            if (u + 1 < nsel) dma_v(u + 1, std::integral_constant<int, 1 - par>{});
        }
    };
    if (!g0) {
        if (1 < nsel) dma_k(1, Odd{});
        dma_v(0, Even{});
        bar();
    }
    auto step = [&](int u, auto par_c) __attribute__((always_inline)) {
        mfma_block(u, par_c);
        dma_wait();
        bar();
        issue_dma(u, par_c);
        softmax_block(u);
        bar();
    };
    step(0, Even{});
    // two tiles per iteration, odd then even, so every stage is a constant
    int u = 1;
    for (; u + 1 < nsel; u += 2) {
        step(u, Odd{});
        step(u + 1, Even{});
    }
    if (u < nsel) step(u++, Odd{});
    // the last P V (u == nsel): V(nsel - 1) is in stage 1 - (nsel & 1)
    if (u & 1) mfma_block(u, Odd{});
    else mfma_block(u, Even{});
    if (g0) bar();

    // ---- O = acc s_v / l; lane holds channels 32 db + 8 r4 + 4 g + [0, 4) ----
    const float la = __shfl(lacc[0], lane & 15, 64), lb = __shfl(lacc[1], lane & 15, 64);
    const float inv = 1.f / (l32 < 16 ? la : lb);
    if (qvalid) {
        uint16_t* op = o + static_cast<int64_t>(q0 + qrow_local) * os + static_cast<int64_t>(head) * kD;
        const float* svp = vsc + (static_cast<int64_t>(seg) * num_heads + head) * kD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = 32 * db + 8 * r4 + 4 * g;
                const f32x4 sv = *reinterpret_cast<const f32x4*>(svp + d);
                u32x2 w;
                w.x = pack_bf16x2(oacc[db][4 * r4 + 0] * (sv.x * inv), oacc[db][4 * r4 + 1] * (sv.y * inv));
                w.y = pack_bf16x2(oacc[db][4 * r4 + 2] * (sv.z * inv), oacc[db][4 * r4 + 3] * (sv.w * inv));
                *reinterpret_cast<u32x2*>(op + d) = w;
            }
    }
    if (skip_counts) {
        if (lane == 0) wskip[wave] = wave_active ? nskip : 0;
        __syncthreads();
        if (tid == 0) {
            int32_t s = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) s += wskip[w];
            skip_counts[item] = s;
        }
    }
}

// Byte offsets of the fp8 scratch (codes, scales, quantise workspace).
struct Fp8Scratch {
    size_t q8, k8, v8t, qsc, ksc, vsc, ws, total;
};

size_t up256(size_t b) { return (b + 255) & ~size_t(255); }

Fp8Scratch fp8_scratch_layout(int num_seqs, int total_tokens, int num_heads) {
    const size_t t = fp8_tiles_upper_bound(num_seqs, total_tokens);
    const size_t hd = static_cast<size_t>(num_heads) * kD;
    Fp8Scratch s;
    size_t off = 0;
    s.q8 = off;  off += up256(static_cast<size_t>(total_tokens) * hd);
    s.k8 = off;  off += up256(t * kBN * hd);
    s.v8t = off; off += up256(t * kBN * hd);
    s.qsc = off; off += up256(t * num_heads * sizeof(float));
    s.ksc = off; off += up256(t * num_heads * sizeof(float));
    s.vsc = off; off += up256(static_cast<size_t>(num_seqs) * hd * sizeof(float));
    s.ws = off;  off += up256(fp8_quant_workspace_bytes(num_seqs, total_tokens, num_heads));
    s.total = off;
    return s;
}

// Block-sparse scratch: the fp8 layout (Q/K codes INT8 there), then the
// code sums and the kept-block lists.
struct BsaScratch {
    Fp8Scratch f;
    size_t qsum, ksum, lists, total;
};

BsaScratch bsa_scratch_layout(int num_seqs, int total_tokens, int num_heads, int64_t list_stride) {
    BsaScratch b;
    b.f = fp8_scratch_layout(num_seqs, total_tokens, num_heads);
    const size_t t = fp8_tiles_upper_bound(num_seqs, total_tokens);
    const size_t sums = up256(t * num_heads * kD * sizeof(int16_t));
    size_t off = b.f.total;
    b.qsum = off;  off += sums;
    b.ksum = off;  off += sums;
    b.lists = off; off += up256(t * num_heads * static_cast<size_t>(list_stride) * sizeof(int32_t));
    b.total = off;
    return b;
}

}  // namespace

size_t bsa_scratch_bytes(int num_seqs, int total_tokens, int num_heads, int64_t list_stride) {
    return bsa_scratch_layout(num_seqs, total_tokens, num_heads, list_stride).total;
}

hipError_t launch_attn_bsa(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           int64_t qs, int64_t ks, int64_t vs, int64_t os, const int32_t* cu,
                           const int32_t* cu_host, const int32_t* items, int64_t num_items,
                           int num_seqs, int total_tokens, int num_heads, float softmax_scale,
                           int sp_permille, int64_t list_stride, int32_t* lists_out, void* scratch,
                           const int32_t* rank_prefix, hipStream_t stream) {
    if (num_items <= 0 || num_seqs <= 0) return hipSuccess;
    int64_t tiles = 0;
    int max_blocks = 0;
    for (int s = 0; s < num_seqs; ++s) {
        const int nb = (cu_host[s + 1] - cu_host[s] + kBN - 1) / kBN;
        tiles += nb;
        max_blocks = nb > max_blocks ? nb : max_blocks;
    }
    const BsaScratch L = bsa_scratch_layout(num_seqs, total_tokens, num_heads, list_stride);
    char* base = static_cast<char*>(scratch);
    uint8_t* q8 = reinterpret_cast<uint8_t*>(base + L.f.q8);
    uint8_t* k8 = reinterpret_cast<uint8_t*>(base + L.f.k8);
    uint8_t* v8t = reinterpret_cast<uint8_t*>(base + L.f.v8t);
    float* qsc = reinterpret_cast<float*>(base + L.f.qsc);
    float* ksc = reinterpret_cast<float*>(base + L.f.ksc);
    float* vsc = reinterpret_cast<float*>(base + L.f.vsc);
    int16_t* qsum = reinterpret_cast<int16_t*>(base + L.qsum);
    int16_t* ksum = reinterpret_cast<int16_t*>(base + L.ksum);
    int32_t* lists = lists_out ? lists_out : reinterpret_cast<int32_t*>(base + L.lists);
    void* ws = base + L.f.ws;
    hipError_t e = launch_fp8_quantize(q, k, v, qs, ks, vs, cu, num_seqs, num_heads, tiles, q8, k8,
                                       v8t, qsc, ksc, vsc, ws, stream, qsum, ksum);
    if (e != hipSuccess) return e;
    const int32_t* tb = static_cast<const int32_t*>(ws);   // tile prefix sums from the quantise pass
    e = launch_bsa_select(qsum, ksum, qsc, ksc, cu, tb, items, num_items, num_seqs, total_tokens,
                          num_heads, tiles, sp_permille, list_stride, lists, max_blocks, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_fp8_kernel<true, false>), dim3(static_cast<unsigned>(num_items)),
                       dim3(kThreads), 0, stream, q8, k8, v8t, qsc, ksc, vsc, o, os, cu, tb,
                       reinterpret_cast<const int4*>(items), num_seqs, total_tokens, num_heads,
                       tiles, softmax_scale * kLog2e, 0.f, nullptr, lists, list_stride, sp_permille,
                       rank_prefix);
    return hipGetLastError();
}

size_t fp8_scratch_bytes(int num_seqs, int total_tokens, int num_heads, int head_dim) {
    if (head_dim != kD) return 0;
    return fp8_scratch_layout(num_seqs, total_tokens, num_heads).total;
}

hipError_t launch_attn_fp8(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           int64_t qs, int64_t ks, int64_t vs, int64_t os, const int32_t* cu,
                           const int32_t* cu_host, const int32_t* items, int64_t num_items,
                           int num_seqs, int total_tokens, int num_heads, int head_dim,
                           float softmax_scale, int skip, float skip_threshold,
                           int32_t* skip_counts, void* scratch, const int32_t* rank_prefix,
                           hipStream_t stream) {
    if (head_dim != kD) return hipErrorInvalidValue;
    if (num_items <= 0 || num_seqs <= 0) return hipSuccess;
    int64_t tiles = 0;
    for (int s = 0; s < num_seqs; ++s) tiles += (cu_host[s + 1] - cu_host[s] + kBN - 1) / kBN;
    const Fp8Scratch L = fp8_scratch_layout(num_seqs, total_tokens, num_heads);
    char* base = static_cast<char*>(scratch);
    uint8_t* q8 = reinterpret_cast<uint8_t*>(base + L.q8);
    uint8_t* k8 = reinterpret_cast<uint8_t*>(base + L.k8);
    uint8_t* v8t = reinterpret_cast<uint8_t*>(base + L.v8t);
    float* qsc = reinterpret_cast<float*>(base + L.qsc);
    float* ksc = reinterpret_cast<float*>(base + L.ksc);
    float* vsc = reinterpret_cast<float*>(base + L.vsc);
    void* ws = base + L.ws;
    hipError_t e = launch_fp8_quantize(q, k, v, qs, ks, vs, cu, num_seqs, num_heads, tiles, q8, k8,
                                       v8t, qsc, ksc, vsc, ws, stream);
    if (e != hipSuccess) return e;
    const int32_t* tb = static_cast<const int32_t*>(ws);   // tile prefix sums from the quantise pass
    const dim3 grid(static_cast<unsigned>(num_items));
    if (skip) {
        hipLaunchKernelGGL((attn_fp8_kernel<false, true>), grid, dim3(kThreads), 0, stream, q8, k8,
                           v8t, qsc, ksc, vsc, o, os, cu, tb, reinterpret_cast<const int4*>(items),
                           num_seqs, total_tokens, num_heads, tiles, softmax_scale * kLog2e,
                           skip_threshold * kLog2e, skip_counts, nullptr, int64_t{0}, 0, rank_prefix);
    } else {
        hipLaunchKernelGGL((attn_fp8_kernel<false, false>), grid, dim3(kThreads), 0, stream, q8, k8,
                           v8t, qsc, ksc, vsc, o, os, cu, tb, reinterpret_cast<const int4*>(items),
                           num_seqs, total_tokens, num_heads, tiles, softmax_scale * kLog2e,
                           skip_threshold * kLog2e, skip_counts, nullptr, int64_t{0}, 0, rank_prefix);
    }
    return hipGetLastError();
}

}  // namespace h3
