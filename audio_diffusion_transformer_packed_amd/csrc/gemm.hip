// bf16 GEMMs on MFMA with the DiT block's fused epilogues ("FastH3 在八卡
// B300 上实现完整 MP4 生成快于播放时长", section "融合 DiT 算子": SwiGLU
// replaces separate SiLU and multiply kernels, and the residual connection
// is fused).
//
//   Store:          y = a . W^T
//   SwiGLU:         y = silu(a . Wg^T) * (a . Wu^T)   (both products in one tile)
//   GatedResidual:  y = res + gate[seg(row)] * (a . W^T)
//
// a: [M, K] bf16 (row stride K); W: [N, K] bf16 (PyTorch [out, in] layout,
// so both operands are contiguous along K). fp32 accumulation; the epilogue
// works on the fp32 accumulator and rounds once to bf16.
//
// Design (CDNA4):
//  * 256 x 256 output tile per workgroup, K step 64, eight waves (two per
//    SIMD, so one wave's LDS waits are covered by the other's MFMAs), each
//    128 activation rows x 64 W rows (2 x 4 blocks of
//    v_mfma_f32_32x32x16_bf16, 128 accumulators per lane);
//  * the MFMA computes C^T = W a^T: the W tile is the A operand, the
//    activation tile the B operand, so each lane ends up owning one output
//    row and four consecutive output columns per register group;
//  * epilogue: each wave stages its 128 x 64 outputs (after the fused
//    operation, rounded to bf16) through 16 KB of LDS, XOR-swizzled, and
//    writes them back row-contiguous with 16-byte stores, 8 lanes per
//    128-byte row segment;
//  * tiles move global -> LDS with buffer_load_dwordx4 ... lds (no staging
//    registers; scalar buffer descriptors, so the loads cost no vector
//    address arithmetic), double buffered; each wave instruction fills 1 KB = 8 rows
//    of 64 bf16, with the 16-byte chunks of row r stored at chunk ^ ((r / 2)
//    % 8): a 16-lane phase of a fragment read (16 consecutive rows, one
//    logical chunk) then covers 2 row parities x 8 chunk slots = all 64
//    banks once (chunk ^ (r % 8) would put rows r and r + 8 on the same banks);
//  * SwiGLU: the W tile interleaves 32-row blocks of Wg and Wu, so each
//    wave's 64 W rows are the gate and up blocks of the same 32 outputs and
//    both accumulators of one output sit in the same lane;
//  * workgroup ids are remapped so each XCD (ids are dealt round-robin over
//    the 8 XCDs) gets a contiguous run of tiles, grouped 4 row-panels at a
//    time, so concurrently running tiles share A and W panels in that XCD's L2.
//
// MXFP8 operands (the same kernel with MX = true; "MiniMax H3 on Ascend
// 950PR / 950DT", section "Recommended lossy configuration": the transformer
// runs with MXFP8 online quantization; the format follows the OCP MX v1.0
// specification): a and W hold E4M3 codes, row-major [rows, K], with one
// E8M0 scale per 32 consecutive K elements of a row, stored K-step-major:
// the scale of row r, block j at byte ((j / 4) rows_total + r) 4 + j % 4, so
// the four scales of a row for one 128-element K step are one aligned dword
// and 32 consecutive rows' dwords are 128 contiguous bytes. A K step is 128
// elements (128 bytes per row, the same LDS tiles and DMA as bf16's 64) and
// runs v_mfma_scale_f32_32x32x64_f8f6f4, which applies the scales inside the
// matrix core. Its operand layout (measured): lane (l, g) (l = lane % 32,
// g = lane / 32) holds 32 bytes of row l; the first 16 bytes of lanes (l, 0)
// and (l, 1) form one 32-element scale block, scaled by the byte selected in
// lane (l, 0)'s scale register, and their last 16 bytes the second block,
// scaled from lane (l, 1). So lane (l, g) reads K elements 16 g + [0, 16)
// and 32 + 16 g + [0, 16) of each 64-element chunk, and its scale register is
// the row's K-step dword shifted right by 8 g, so that byte 2c holds block
// 2c + g of chunk c. The SwiGLU epilogue then writes its output as MXFP8
// (codes and scales in the same layouts), ready for the down projection.
#include <type_traits>

#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {
namespace {

constexpr int kBM = 256;          // activation rows per tile
constexpr int kBN = 256;          // W rows per tile (output columns, or gate+up pairs)
constexpr int kStepBytes = 128;   // bytes of a row per K step (64 bf16 or 128 fp8)
constexpr int kWaves = 8;         // two per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kWN = 2;            // 32-row W blocks per wave (64 output columns, or one gate+up pair)
constexpr int kWM = 4;            // 32-row activation blocks per wave (128 rows)
constexpr int kDmaPerWave = kBM / 8 / kWaves;   // 1 KB DMA instructions per wave and operand
constexpr int kTileBytes = kBM * kStepBytes;   // 32 KB per operand tile
constexpr int kStageBytes = 2 * kTileBytes;    // W tile then activation tile
constexpr int kGroupM = 4;
constexpr int kXcds = 8;

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

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 4 bytes per lane from buffer offset voff + soff into LDS at lds_dst + 4 i.
__device__ __forceinline__ void buf_dma4(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, int soff,
                                         void* lds_dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(lds_dst)),
        4, voff, soff, 0, 0);
}

// Scaled fp8 MFMA; OP selects the byte of each lane's scale register.
template <int OP>
__device__ __forceinline__ f32x16 mfma_mx(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OP, sa, OP, sb);
}

// MXFP4 operands (E2M1, cbsz = blgp = 4): 32 elements (16 bytes) per lane,
// the low half of the operand registers.
template <int OP>
__device__ __forceinline__ f32x16 mfma_mx4(uint4 a, uint4 b, f32x16 c, int sa, int sb) {
    const i32x8 av = {static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z),
                      static_cast<int>(a.w), 0, 0, 0, 0};
    const i32x8 bv = {static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z),
                      static_cast<int>(b.w), 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, OP, sa, OP, sb);
}

__device__ __forceinline__ i32x8 cat16(uint4 x, uint4 y) {
    return i32x8{static_cast<int>(x.x), static_cast<int>(x.y), static_cast<int>(x.z), static_cast<int>(x.w),
                 static_cast<int>(y.x), static_cast<int>(y.y), static_cast<int>(y.z), static_cast<int>(y.w)};
}

struct GemmArgs {
    const void* a;            // [M, K] bf16, or E4M3 codes
    const void* w;            // [N, K]
    const void* w2;           // [N, K] up matrix (SwiGLU)
    const uint8_t* a_sc;      // MX scales of a, w, w2 (K-step-major)
    const uint8_t* w_sc;
    const uint8_t* w2_sc;
    void* y;                  // [M, N] bf16, or E4M3 codes (SwiGLU with MX)
    uint8_t* y_sc;            // MX scales of y (SwiGLU with MX)
    int64_t M, N, K;
    const uint16_t* res;      // gated residual
    const float* gate;
    int64_t gate_stride;
    const int32_t* cu;
    int num_seqs;
    int mtiles, ntiles;
};

// Tile id -> (row panel, column panel), XCD-aware and grouped.
__device__ __forceinline__ void tile_coords(int bid, int nblocks, int mt, int nt, int& tm, int& tn) {
    // contiguous run per XCD (block b runs on XCD b % 8); XCD x owns
    // per + (x < rem) consecutive tiles starting at x * per + min(x, rem)
    const int per = nblocks / kXcds, rem = nblocks % kXcds;
    const int xcd = bid % kXcds;
    const int t = xcd * per + min(xcd, rem) + bid / kXcds;
    const int group = t / (kGroupM * nt);
    const int first_m = group * kGroupM;
    const int gm = min(kGroupM, mt - first_m);
    const int w = t - group * kGroupM * nt;
    tm = first_m + w % gm;
    tn = w / gm;
}

// operand formats
constexpr int kFmtBf16 = 0, kFmtFp8 = 1, kFmtFp4 = 2;

template <int EPI, int FMT>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmArgs p) {
    constexpr bool MX = FMT != kFmtBf16;
    constexpr bool FP4 = FMT == kFmtFp4;
    // scale bytes per row and K step: 4 E8M0 bytes (fp8), 8 (fp4)
    constexpr int kSB = FP4 ? 8 : 4;
    __shared__ __attribute__((aligned(1024))) char smem[2 * (kStageBytes + (MX ? 256 * kSB * 2 : 0))];
    const char* __restrict__ A = static_cast<const char*>(p.a);
    const char* __restrict__ W = static_cast<const char*>(p.w);
    const char* __restrict__ W2 = static_cast<const char*>(p.w2);
    const int64_t M = p.M, N = p.N, K = p.K;
    const uint16_t* __restrict__ res = p.res;
    const float* __restrict__ gate = p.gate;
    const int64_t gate_stride = p.gate_stride;
    const int32_t* __restrict__ cu = p.cu;
    const int num_seqs = p.num_seqs, mtiles = p.mtiles, ntiles = p.ntiles;
    uint16_t* __restrict__ Y = static_cast<uint16_t*>(p.y);
    // bytes per operand row: bf16 2, fp8 1, fp4 1/2 per element
    const int64_t row_bytes = FP4 ? K / 2 : (MX ? K : 2 * K);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int wn = wave >> 1;     // W-tile rows 64 wn .. 64 wn + 63
    const int wm = wave & 1;      // activation rows 128 wm .. 128 wm + 127

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, mtiles, ntiles, tm, tn);
    const int64_t m0 = static_cast<int64_t>(tm) * kBM;
    constexpr int OUT_N = EPI == kEpiSwiGLU ? kBN / 2 : kBN;
    const int64_t n0 = static_cast<int64_t>(tn) * OUT_N;

    // ---- DMA: wave w fills tile rows 64 w + 8 i + lane/8 (i = 0..7); the
    // lane's LDS slot is physical chunk lane % 8, which holds logical chunk
    // (lane % 8) ^ ((row / 2) % 8). Buffer descriptors based at the tile's
    // first row live in scalar registers and are sized to the rows that
    // exist: rows past M (or N) are out of range and load as zeros (their
    // outputs are never stored). Per lane only a constant byte offset is
    // kept; the K position is the scalar offset of each load.
    const int rl = lane >> 3;
    const int64_t a_rows = min<int64_t>(kBM, M - m0);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(A + m0 * row_bytes), 0, static_cast<int>(a_rows * row_bytes), kBufferWord3);
    constexpr int W_ROWS = EPI == kEpiSwiGLU ? kBN / 2 : kBN;   // W rows per operand matrix
    const int64_t w_rows = min<int64_t>(W_ROWS, N - n0);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(W + n0 * row_bytes), 0, static_cast<int>(w_rows * row_bytes), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rw2 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>((EPI == kEpiSwiGLU ? W2 : W) + n0 * row_bytes), 0,
        static_cast<int>(w_rows * row_bytes), kBufferWord3);
    uint32_t aoff[kDmaPerWave], woff[kDmaPerWave];
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
        const int r = 8 * kDmaPerWave * wave + 8 * i + rl;     // tile row
        const int chunk = (lane & 7) ^ ((r >> 1) & 7);
        aoff[i] = static_cast<uint32_t>(r * row_bytes + 16 * chunk);
        if (EPI == kEpiSwiGLU) {
            // W-tile row r = 128 wnp + 32 bj + j: bj even -> gate (W), odd -> up
            // (W2), for output column n0 + 64 wnp + 32 (bj / 2) + j; a wave's
            // rows share one bj (r / 32 = wave), so the matrix is wave-uniform
            const int wnp = r >> 7, bj = (r >> 5) & 3, j = r & 31;
            woff[i] = static_cast<uint32_t>((64 * wnp + 32 * (bj >> 1) + j) * row_bytes + 16 * chunk);
        } else {
            woff[i] = static_cast<uint32_t>(r * row_bytes + 16 * chunk);
        }
    }

    // MX scales ride with the tiles: per K step the 256 activation rows'
    // dwords (1 KB, contiguous in the K-step-major layout) and the 256 W
    // rows' dwords (for SwiGLU 128 gate rows then 128 up rows) are DMA'd
    // into 2 KB after the two tiles of the stage, by waves 0 and 1. Scale
    // rows past the matrix read past-the-end zeros or the next K step's
    // first rows; their data rows load as zeros and are never stored.
    const int64_t ks_total = row_bytes / kStepBytes;
    const int sa_bytes = MX ? static_cast<int>((ks_total * M - m0) * kSB) : 0;
    const int sw_bytes = MX ? static_cast<int>((ks_total * N - n0) * kSB) : 0;
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.a_sc) + (MX ? m0 * kSB : 0), 0, sa_bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rsw1 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.w_sc) + (MX ? n0 * kSB : 0), 0, sw_bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rsw2 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(EPI == kEpiSwiGLU ? p.w2_sc : p.w_sc) + (MX ? n0 * kSB : 0), 0, sw_bytes,
        kBufferWord3);
    // per stage: the W rows' scale records, then the activation rows'
    constexpr int kScaleBytes = MX ? 2 * 256 * kSB : 0;
    constexpr int kStage = kStageBytes + kScaleBytes;

    // per-wave constant sources (selected once, so they stay in scalar registers)
    const bool up = EPI == kEpiSwiGLU && (wave & 1);
    const __amdgpu_buffer_rsrc_t rwx = up ? rw2 : rw;
    // MX scales: every wave moves 256 B per K step (4 per lane, no branch):
    // waves 0-3 the W rows' dwords (SwiGLU: waves 0-1 gate rows, 2-3 up
    // rows), waves 4-7 the activation rows'
    // MXFP4: 8-byte records, 16 B per lane; waves 0-1 the W rows' 2 KB
    // (SwiGLU: wave 0 the gate rows, wave 1 the up rows), waves 2-3 the
    // activation rows', waves 4-7 none
    const bool wpart = FP4 ? wave < 2 : wave < 4;
    const __amdgpu_buffer_rsrc_t rsx =
        FP4 ? (wpart ? ((EPI == kEpiSwiGLU && wave == 1) ? rsw2 : rsw1) : rsa)
            : (wpart ? ((EPI == kEpiSwiGLU && wave >= 2) ? rsw2 : rsw1) : rsa);
    const uint32_t sc_voff =
        FP4 ? static_cast<uint32_t>(16 * lane + ((EPI == kEpiSwiGLU && wpart) ? 0 : 1024 * (wave & 1)))
            : static_cast<uint32_t>(4 * (64 * (EPI == kEpiSwiGLU && wpart ? (wave & 1) : (wave & 3)) + lane));
    const int64_t sc_rows = wpart ? N : M;

    auto issue = [&](int stage, int64_t kt) __attribute__((always_inline)) {
        char* base = smem + stage * kStage;
        const int kb = static_cast<int>(kt * kStepBytes);
#pragma unroll
        for (int i = 0; i < kDmaPerWave; ++i) {
            buf_dma16(rwx, woff[i], kb, base + (kDmaPerWave * wave + i) * 1024);
            buf_dma16(ra, aoff[i], kb, base + kTileBytes + (kDmaPerWave * wave + i) * 1024);
        }
        if constexpr (FP4) {
            if (wave < 4)
                buf_dma16(rsx, sc_voff, static_cast<int>(kt * sc_rows * 8), base + kStageBytes + 1024 * wave);
        } else if constexpr (MX) {
            buf_dma4(rsx, sc_voff, static_cast<int>(kt * sc_rows * 4), base + kStageBytes + 256 * wave);
        }
    };
    // this lane's scale dwords in a stage (shifted by 8 g, see the header)
    uint32_t asc[kWM], wsc[kWN];
    auto take_scales = [&](int stage) __attribute__((always_inline)) {
        const uint32_t* sw = reinterpret_cast<const uint32_t*>(smem + stage * kStage + kStageBytes);
        if constexpr (FP4) {
            // record of a row: dword g holds the blocks g, g + 2, g + 4, g + 6
            // of the step, which this lane's MFMAs of chunks 0..3 take
            const uint32_t* sa = sw + 512;
#pragma unroll
            for (int b = 0; b < kWM; ++b) asc[b] = sa[2 * (128 * wm + 32 * b + l32) + g];
#pragma unroll
            for (int b = 0; b < kWN; ++b)
                wsc[b] = sw[2 * (EPI == kEpiSwiGLU ? 128 * b + 32 * wn + l32 : 64 * wn + 32 * b + l32) + g];
            return;
        }
        const uint32_t* sa = sw + 256;
#pragma unroll
        for (int b = 0; b < kWM; ++b) asc[b] = sa[128 * wm + 32 * b + l32] >> (8 * g);
#pragma unroll
        for (int b = 0; b < kWN; ++b)
            wsc[b] = sw[EPI == kEpiSwiGLU ? 128 * b + 32 * wn + l32 : 64 * wn + 32 * b + l32] >> (8 * g);
    };

    f32x16 acc[kWN][kWM];
#pragma unroll
    for (int i = 0; i < kWN; ++i)
#pragma unroll
        for (int j = 0; j < kWM; ++j) acc[i][j] = f32x16{};

    // fragment read offsets: row R (tile row), chunk c -> R * 128 + 16 * (c ^ ((R / 2) % 8))
    // rows used by this lane: 128 w* + 32 b + l32, so (R / 2) % 8 == (l32 / 2) % 8
    const int rsw = (l32 >> 1) & 7;
    const int wrow0 = (64 * wn + l32) * 128;
    const int arow0 = (128 * wm + l32) * 128;

    const int64_t ksteps = ks_total;
    issue(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int64_t kt = 0; kt < ksteps; ++kt) {
        const int stage = static_cast<int>(kt & 1);
        if (MX) take_scales(stage);
        if (kt + 1 < ksteps) issue(stage ^ 1, kt + 1);
        const char* wt = smem + stage * kStage;
        const char* at = wt + kTileBytes;
        if constexpr (FP4) {
            // four 64-element chunks c (32 bytes of a row each): lane (l, g)
            // reads 16-byte chunk 2c + g, the 32 elements of block 2c + g,
            // scaled by byte c of its scale dword
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int off = 16 * ((2 * c + g) ^ rsw);
                bf16x8 wf[kWN], af[kWM];
#pragma unroll
                for (int b = 0; b < kWN; ++b) wf[b] = *reinterpret_cast<const bf16x8*>(wt + wrow0 + b * 32 * 128 + off);
#pragma unroll
                for (int b = 0; b < kWM; ++b) af[b] = *reinterpret_cast<const bf16x8*>(at + arow0 + b * 32 * 128 + off);
#pragma unroll
                for (int bi = 0; bi < kWN; ++bi)
#pragma unroll
                    for (int bj = 0; bj < kWM; ++bj) {
                        const uint4 wa = __builtin_bit_cast(uint4, wf[bi]);
                        const uint4 aa = __builtin_bit_cast(uint4, af[bj]);
                        const int sw = static_cast<int>(wsc[bi]), sa = static_cast<int>(asc[bj]);
                        switch (c) {
                            case 0: acc[bi][bj] = mfma_mx4<0>(wa, aa, acc[bi][bj], sw, sa); break;
                            case 1: acc[bi][bj] = mfma_mx4<1>(wa, aa, acc[bi][bj], sw, sa); break;
                            case 2: acc[bi][bj] = mfma_mx4<2>(wa, aa, acc[bi][bj], sw, sa); break;
                            default: acc[bi][bj] = mfma_mx4<3>(wa, aa, acc[bi][bj], sw, sa); break;
                        }
                    }
            }
        } else if constexpr (MX) {
            // two 64-element chunks c: lane reads 16-byte chunks 4c + g and
            // 4c + 2 + g. The fragments are read as bf16x8 (reinterpreted as
            // fp8 bytes): read as uint4 the compiler could not tell them from
            // the in-flight DMA's LDS writes and waited for the DMA first.
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int o0 = 16 * ((4 * c + g) ^ rsw), o1 = 16 * ((4 * c + 2 + g) ^ rsw);
                bf16x8 w0[kWN], w1[kWN], a0[kWM], a1[kWM];
#pragma unroll
                for (int b = 0; b < kWN; ++b) w0[b] = *reinterpret_cast<const bf16x8*>(wt + wrow0 + b * 32 * 128 + o0);
#pragma unroll
                for (int b = 0; b < kWN; ++b) w1[b] = *reinterpret_cast<const bf16x8*>(wt + wrow0 + b * 32 * 128 + o1);
#pragma unroll
                for (int b = 0; b < kWM; ++b) a0[b] = *reinterpret_cast<const bf16x8*>(at + arow0 + b * 32 * 128 + o0);
#pragma unroll
                for (int b = 0; b < kWM; ++b) a1[b] = *reinterpret_cast<const bf16x8*>(at + arow0 + b * 32 * 128 + o1);
#pragma unroll
                for (int bi = 0; bi < kWN; ++bi)
#pragma unroll
                    for (int bj = 0; bj < kWM; ++bj) {
                        const i32x8 wa = cat16(__builtin_bit_cast(uint4, w0[bi]), __builtin_bit_cast(uint4, w1[bi]));
                        const i32x8 aa = cat16(__builtin_bit_cast(uint4, a0[bj]), __builtin_bit_cast(uint4, a1[bj]));
                        const int sw = static_cast<int>(wsc[bi]), sa = static_cast<int>(asc[bj]);
                        acc[bi][bj] = c == 0 ? mfma_mx<0>(wa, aa, acc[bi][bj], sw, sa)
                                             : mfma_mx<2>(wa, aa, acc[bi][bj], sw, sa);
                    }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int off = 16 * ((2 * ks + g) ^ rsw);
                bf16x8 wf[kWN], af[kWM];
#pragma unroll
                for (int b = 0; b < kWN; ++b) wf[b] = *reinterpret_cast<const bf16x8*>(wt + wrow0 + b * 32 * 128 + off);
#pragma unroll
                for (int b = 0; b < kWM; ++b) af[b] = *reinterpret_cast<const bf16x8*>(at + arow0 + b * 32 * 128 + off);
#pragma unroll
                for (int bi = 0; bi < kWN; ++bi)
#pragma unroll
                    for (int bj = 0; bj < kWM; ++bj) acc[bi][bj] = mfma32x32x16(wf[bi], af[bj], acc[bi][bj]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- epilogue through LDS. acc[bi][bj] register 4 q + e holds output
    // row 128 wm + 32 bj + l32 of the tile and W-tile row 64 wn + 32 bi +
    // 8 q + 4 g + e, so a lane owns one row and a wave store would write 8
    // bytes into each of 32 rows (one L2 write request per 16 bytes). Each
    // wave instead stages its own 128 x 64 outputs in 16 KB of the (now
    // free) stage buffers, 16-byte chunks of row r XOR-swizzled by r / 2,
    // and reads them back row-contiguous, so 8 (or 4) lanes write a row's
    // 128 (64) bytes together with 16-byte stores. The staging is
    // wave-local: only this wave's LDS accesses need ordering.
    char* ep = smem + wave * (2 * kStageBytes / kWaves);
    const bool vec16 = ((reinterpret_cast<uintptr_t>(p.y) | reinterpret_cast<uintptr_t>(res)) & 15) == 0;
    auto lds_fence = []() __attribute__((always_inline)) { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };
    auto store8 = [&](uint16_t* dst, uint4 v) __attribute__((always_inline)) {
        if (vec16) {
            *reinterpret_cast<uint4*>(dst) = v;
        } else {
            reinterpret_cast<uint2*>(dst)[0] = make_uint2(v.x, v.y);
            reinterpret_cast<uint2*>(dst)[1] = make_uint2(v.z, v.w);
        }
    };
    const int64_t mw = m0 + 128 * wm;        // first row of this wave's outputs
    if (EPI == kEpiStore) {
        // 128 rows x 64 bf16 (128 B) per wave
#pragma unroll
        for (int bj = 0; bj < kWM; ++bj) {
            const int r = 32 * bj + l32;
#pragma unroll
            for (int bi = 0; bi < kWN; ++bi)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = 4 * bi + q;
                    u32x2 w;
                    w.x = pack_bf16x2(acc[bi][bj][4 * q], acc[bi][bj][4 * q + 1]);
                    w.y = pack_bf16x2(acc[bi][bj][4 * q + 2], acc[bi][bj][4 * q + 3]);
                    *reinterpret_cast<u32x2*>(ep + r * 128 + 16 * (c ^ ((r >> 1) & 7)) + 8 * g) = w;
                }
        }
        lds_fence();
        const int64_t n = n0 + 64 * wn + 8 * (lane & 7);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int r = 8 * j + (lane >> 3);
            const uint4 v = *reinterpret_cast<const uint4*>(ep + r * 128 + 16 * ((lane & 7) ^ ((r >> 1) & 7)));
            if (mw + r < M && n < N) store8(Y + (mw + r) * N + n, v);
        }
    } else if (EPI == kEpiSwiGLU && FMT == kFmtFp8) {
        // bi = 0 is the gate block, bi = 1 the up block of output columns
        // n0 + 32 wn + [0, 32), exactly one MX block per row: fp32 staging
        // (128 rows x 32 fp32 per wave), then 4 lanes per row take the
        // block's amax, scale byte and E4M3 codes (8 per lane)
#pragma unroll
        for (int bj = 0; bj < kWM; ++bj) {
            const int r = 32 * bj + l32;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float gv = acc[0][bj][4 * q + e];
                    const float uv = acc[1][bj][4 * q + e];
                    o[e] = gv / (1.0f + __expf(-gv)) * uv;
                }
                *reinterpret_cast<f32x4*>(ep + r * 128 + 16 * ((2 * q + g) ^ ((r >> 1) & 7))) = o;
            }
        }
        lds_fence();
        uint8_t* Y8 = static_cast<uint8_t*>(p.y);
        const int64_t n = n0 + 32 * wn + 8 * (lane & 3);
        const int64_t blk = (n0 + 32 * wn) >> 5;           // MX block of this wave's columns
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 16 * j + (lane >> 2);
            const f32x4 lo = *reinterpret_cast<const f32x4*>(ep + r * 128 + 16 * ((2 * (lane & 3)) ^ ((r >> 1) & 7)));
            const f32x4 hi = *reinterpret_cast<const f32x4*>(ep + r * 128 + 16 * ((2 * (lane & 3) + 1) ^ ((r >> 1) & 7)));
            float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            float am = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
            am = fmaxf(am, __shfl_xor(am, 1, 64));
            am = fmaxf(am, __shfl_xor(am, 2, 64));
            const uint32_t sb = mx_scale_byte(am);
            const float inv = mx_inv_scale(sb);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] *= inv;
            const uint2 codes = mx_codes8(v);
            const int64_t m = mw + r;
            if (m < M && n < N) {
                *reinterpret_cast<uint2*>(Y8 + m * N + n) = codes;
                if ((lane & 3) == 0) p.y_sc[((blk >> 2) * M + m) * 4 + (blk & 3)] = static_cast<uint8_t>(sb);
            }
        }
    } else if (EPI == kEpiSwiGLU) {
        // bi = 0 is the gate block, bi = 1 the up block of output columns
        // n0 + 32 wn + [0, 32): 128 rows x 32 bf16 (64 B) per wave
#pragma unroll
        for (int bj = 0; bj < kWM; ++bj) {
            const int r = 32 * bj + l32;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float gv = acc[0][bj][4 * q + e];
                    const float uv = acc[1][bj][4 * q + e];
                    o[e] = gv / (1.0f + __expf(-gv)) * uv;
                }
                u32x2 w;
                w.x = pack_bf16x2(o[0], o[1]);
                w.y = pack_bf16x2(o[2], o[3]);
                *reinterpret_cast<u32x2*>(ep + r * 64 + 16 * (q ^ ((r >> 2) & 3)) + 8 * g) = w;
            }
        }
        lds_fence();
        const int64_t n = n0 + 32 * wn + 8 * (lane & 3);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 16 * j + (lane >> 2);
            const uint4 v = *reinterpret_cast<const uint4*>(ep + r * 64 + 16 * ((lane & 3) ^ ((r >> 2) & 3)));
            if (mw + r < M && n < N) store8(Y + (mw + r) * N + n, v);
        }
    } else {
        // y = res + gate[seg] * acc, rounded once: fp32 staging, one 32-column
        // block (bi) at a time, 128 rows x 32 fp32 (128 B) per wave
        int segs[kWM];
#pragma unroll
        for (int bj = 0; bj < kWM; ++bj) {
            const int64_t m = mw + 32 * bj + l32;
            segs[bj] = (num_seqs > 1 && m < M) ? find_segment(cu, num_seqs, m) : 0;
        }
#pragma unroll
        for (int bi = 0; bi < kWN; ++bi) {
            if (bi > 0) lds_fence();       // previous block's reads are done before it is overwritten
#pragma unroll
            for (int bj = 0; bj < kWM; ++bj) {
                const int r = 32 * bj + l32;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = 2 * q + g;
                    f32x4 v = {acc[bi][bj][4 * q], acc[bi][bj][4 * q + 1], acc[bi][bj][4 * q + 2],
                               acc[bi][bj][4 * q + 3]};
                    *reinterpret_cast<f32x4*>(ep + r * 128 + 16 * (c ^ ((r >> 1) & 7))) = v;
                }
            }
            lds_fence();
            const int64_t n = n0 + 64 * wn + 32 * bi + 8 * (lane & 3);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 16 * j + (lane >> 2);
                // rows 16 j .. 16 j + 15 lie in 32-row block j / 2
                const int seg = num_seqs > 1 ? __shfl(segs[j >> 1], r & 31, 64) : 0;
                const f32x4 lo = *reinterpret_cast<const f32x4*>(ep + r * 128 + 16 * ((2 * (lane & 3)) ^ ((r >> 1) & 7)));
                const f32x4 hi = *reinterpret_cast<const f32x4*>(ep + r * 128 + 16 * ((2 * (lane & 3) + 1) ^ ((r >> 1) & 7)));
                const int64_t m = mw + r;
                if (m < M && n < N) {
                    uint4 rv;
                    if (vec16) {
                        rv = *reinterpret_cast<const uint4*>(res + m * N + n);
                    } else {
                        const uint2 r0 = reinterpret_cast<const uint2*>(res + m * N + n)[0];
                        const uint2 r1 = reinterpret_cast<const uint2*>(res + m * N + n)[1];
                        rv = make_uint4(r0.x, r0.y, r1.x, r1.y);
                    }
                    const f32x4 g0 = *reinterpret_cast<const f32x4*>(gate + seg * gate_stride + n);
                    const f32x4 g1 = *reinterpret_cast<const f32x4*>(gate + seg * gate_stride + n + 4);
                    const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
                    const float a8[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    const float g8[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
                    uint32_t ow[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const float x0 = fmaf(g8[2 * p], a8[2 * p], __uint_as_float(rw[p] << 16));
                        const float x1 = fmaf(g8[2 * p + 1], a8[2 * p + 1], __uint_as_float(rw[p] & 0xffff0000u));
                        ow[p] = pack_bf16x2(x0, x1);
                    }
                    store8(Y + m * N + n, make_uint4(ow[0], ow[1], ow[2], ow[3]));
                }
            }
        }
    }
}

template <int FMT>
hipError_t launch_gemm_args(int epilogue, GemmArgs& p, hipStream_t stream) {
    if (p.M == 0) return hipSuccess;
    const int out_n = epilogue == kEpiSwiGLU ? kBN / 2 : kBN;
    p.mtiles = static_cast<int>((p.M + kBM - 1) / kBM);
    p.ntiles = static_cast<int>((p.N + out_n - 1) / out_n);
    const dim3 grid(static_cast<unsigned>(p.mtiles * p.ntiles));
    switch (epilogue) {
        case kEpiStore:
            hipLaunchKernelGGL((gemm_kernel<kEpiStore, FMT>), grid, dim3(kThreads), 0, stream, p);
            break;
        case kEpiSwiGLU:
            hipLaunchKernelGGL((gemm_kernel<kEpiSwiGLU, FMT>), grid, dim3(kThreads), 0, stream, p);
            break;
        default:
            hipLaunchKernelGGL((gemm_kernel<kEpiGatedResidual, FMT>), grid, dim3(kThreads), 0, stream, p);
            break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int epilogue, const uint16_t* a, const uint16_t* w, const uint16_t* w2,
                       uint16_t* y, int64_t m, int64_t n, int64_t k, const uint16_t* res,
                       const float* gate, int64_t gate_stride, const int32_t* cu,
                       int num_seqs, hipStream_t stream) {
    GemmArgs p{};
    p.a = a; p.w = w; p.w2 = w2; p.y = y;
    p.M = m; p.N = n; p.K = k;
    p.res = res; p.gate = gate; p.gate_stride = gate_stride; p.cu = cu; p.num_seqs = num_seqs;
    return launch_gemm_args<kFmtBf16>(epilogue, p, stream);
}

hipError_t launch_gemm_mx(int epilogue, const uint8_t* a, const uint8_t* a_sc, const uint8_t* w,
                          const uint8_t* w_sc, const uint8_t* w2, const uint8_t* w2_sc, void* y,
                          uint8_t* y_sc, int64_t m, int64_t n, int64_t k, const uint16_t* res,
                          const float* gate, int64_t gate_stride, const int32_t* cu, int num_seqs,
                          hipStream_t stream) {
    GemmArgs p{};
    p.a = a; p.a_sc = a_sc; p.w = w; p.w_sc = w_sc; p.w2 = w2; p.w2_sc = w2_sc;
    p.y = y; p.y_sc = y_sc;
    p.M = m; p.N = n; p.K = k;
    p.res = res; p.gate = gate; p.gate_stride = gate_stride; p.cu = cu; p.num_seqs = num_seqs;
    return launch_gemm_args<kFmtFp8>(epilogue, p, stream);
}

hipError_t launch_gemm_mx4(int epilogue, const uint8_t* a, const uint8_t* a_sc, const uint8_t* w,
                           const uint8_t* w_sc, const uint8_t* w2, const uint8_t* w2_sc, void* y,
                           int64_t m, int64_t n, int64_t k, const uint16_t* res, const float* gate,
                           int64_t gate_stride, const int32_t* cu, int num_seqs, hipStream_t stream) {
    GemmArgs p{};
    p.a = a; p.a_sc = a_sc; p.w = w; p.w_sc = w_sc; p.w2 = w2; p.w2_sc = w2_sc;
    p.y = y;
    p.M = m; p.N = n; p.K = k;
    p.res = res; p.gate = gate; p.gate_stride = gate_stride; p.cu = cu; p.num_seqs = num_seqs;
    return launch_gemm_args<kFmtFp4>(epilogue, p, stream);
}

}  // namespace h3
