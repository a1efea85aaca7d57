// fp8 (OCP e4m3fn) quantisation of packed Q, K and V for the fp8 attention
// path ("MiniMax H3 FastH3 real-time serving with vLLM-Omni", section
// "Scaling beyond the FastH3 profile", sparse & quantized attention bullet:
// SAGE runs attention in FP8; "FastH3 在八卡 B300 上实现完整 MP4 生成快于播放时长",
// section "其他加速路径：有损但可控").
//
// The pages name FP8 attention but not its granularity; this follows one
// reading: Q and K get one scale per (head, 64-token block aligned to the
// segment start), V one scale per (segment, head, channel); scale = amax /
// 448 (1 when amax is 0) and code = e4m3(x / scale), round to nearest even,
// clamped to +-448, with the scale taken exactly: code = RNE(448 x / amax).
//
// The code decision is exact without a division per element. For bf16 x
// and amax, 448 x has at most 11 significant bits, amax at most 8, and an
// e4m3 rounding midpoint m at most 5, so 448 x - m amax is either 0 (the
// quotient is on the midpoint) or a nonzero multiple of the smaller of the
// two products' last-place units; both products have integer significands
// below 255 * 31 = 7905, so the quotient then lies more than 2^-13
// (relative) from m. The product x * fl(448 / amax) is within 2^-23 of
// the quotient; rounding it to 16 significant bits (fp8_snap: half a step is
// 2^-16) lands exactly on m in the first case and stays on the quotient's
// side of m in the second, so the hardware's round-to-nearest-even
// conversion of the snapped value gives the code of the exact quotient
// (ties to even included). Since |x| <= amax the snapped value never exceeds
// 448, so no clamp is needed. Blocks with amax < 2^-64 scale x and amax by
// 2^64 first (exact) so that 448 / amax stays finite.
//
// Layouts written (T = sum over segments of ceil(L_s / 64), the key tiles):
//   q8   [N, H, 128]        token-major, like q;
//   k8   [H, T, 64, 128]    key tiles of 64 tokens; rows past a segment's end
//                           are 0, so a tile is one contiguous 8 KB block;
//   v8t  [H, T, 128, 64]    V transposed per key tile (channel-major, keys
//                           contiguous), keys permuted inside the tile: key
//                           32b + 8i + 4g + e (b, g in {0,1}; i, e in 0..3)
//                           sits at position 32g + 16b + 4i + e, the order
//                           in which the attention kernel's lanes hold P;
//   q_scale, k_scale [T, H];  v_scale [B, H, 128].
// With code sums requested (the block-sparse path) Q and K are INT8 instead:
// scale = amax / 127 (1 when amax is 0), code = round-half-even(127 x /
// amax) in [-127, 127], same layouts, plus per (tile, head) the per-channel
// sums of the Q codes (qsum [T, H, 128]) and of the K codes (ksum [H, 16,
// T, 8]: channel chunk-major, so that consecutive key blocks' 16-byte chunks
// are adjacent), int16 (|sum| <= 64 * 127), the block means the block
// selection ranks by.
// All HBM-bound: q and k are streamed once by one quant_qk_kernel launch
// each, v twice, by vamax_kernel (its per-tile channel amax) and by
// quant_v_kernel (V's scale needs the whole segment first), with 16-byte
// nontemporal loads. One tensor per launch keeps one tile in registers
// (46-52 VGPRs, eight waves per SIMD): Q and K together in one kernel
// (86 VGPRs, five waves) measured 2 % slower over the pass, and with V's
// amax folded in as well (97 VGPRs, four waves) 4 % slower. Work items are ordered head-fastest, so the
// workgroups resident at one time read whole token rows. Q and K codes are
// stored nontemporally; V code rows are 64 bytes, half a cache line, so
// they are stored through L2, which merges the two halves before write-back
// (nontemporal stores there measured 15 % slower).
#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {
namespace {

constexpr int kD = 128;          // head dim of the fp8 path
constexpr int kTB = 64;          // tokens per Q/K scale block and per key tile
constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float fp8_scale_of(float amax) {
    return amax > 0.f ? amax / kE4M3Max : 1.0f;
}

// x -> 448 x / amax as (x * pre) * mul, see the header comment. amax == 0
// means every x of the block is 0, and any finite mul gives code 0.
struct Fp8Mul {
    float pre, mul;
};
__device__ __forceinline__ Fp8Mul fp8_mul_of(float amax) {
    const float pre = amax < 0x1p-64f ? 0x1p64f : 1.0f;
    return {pre, amax > 0.f ? kE4M3Max / (amax * pre) : 0.f};
}

// Round to 16 significant bits, ties away from zero (integer add on the
// magnitude bits; the sign bit is untouched for finite values).
__device__ __forceinline__ float fp8_snap(float y) {
    return __uint_as_float((__float_as_uint(y) + 0x80u) & ~0xffu);
}

__device__ __forceinline__ float fp8_prep(float x, Fp8Mul m) { return fp8_snap((x * m.pre) * m.mul); }

// Codes of a and b into bytes 0, 1 (Hi = false) or 2, 3 (Hi = true) of `old`.
template <bool Hi>
__device__ __forceinline__ uint32_t e4m3x2(float a, float b, uint32_t old) {
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, static_cast<int>(old), Hi));
}

// Codes of the eight values of a bf16 chunk, byte j = value j.
__device__ __forceinline__ u32x2 codes8(uint4 raw, Fp8Mul m) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    u32x2 out;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const uint32_t lo = w[2 * p], hi = w[2 * p + 1];
        uint32_t c = e4m3x2<false>(fp8_prep(__uint_as_float(lo << 16), m),
                                   fp8_prep(__uint_as_float(lo & 0xffff0000u), m), 0u);
        c = e4m3x2<true>(fp8_prep(__uint_as_float(hi << 16), m),
                         fp8_prep(__uint_as_float(hi & 0xffff0000u), m), c);
        out[p] = c;
    }
    return out;
}

__device__ __forceinline__ float absmax8(uint4 raw) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float m = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p)
        m = fmaxf(m, fmaxf(fabsf(__uint_as_float(w[p] << 16)), fabsf(__uint_as_float(w[p] & 0xffff0000u))));
    return m;
}

// Value j (0..7) of a bf16 chunk as fp32.
__device__ __forceinline__ float chunk_val(uint4 raw, int j) {
    const uint32_t w = j < 2 ? raw.x : j < 4 ? raw.y : j < 6 ? raw.z : raw.w;
    return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
}

// tb[s] = sum_{r < s} ceil(L_r / 64), tb[B] = T. One workgroup.
__global__ __launch_bounds__(1024) void tile64_scan_kernel(const int32_t* __restrict__ cu, int num_seqs,
                                                           int32_t* __restrict__ tb) {
    __shared__ int32_t part[1024];
    const int tid = threadIdx.x;
    const int per = (num_seqs + 1023) / 1024;
    const int s0 = min(num_seqs, tid * per), s1 = min(num_seqs, s0 + per);
    int32_t sum = 0;
    for (int s = s0; s < s1; ++s) sum += (max(0, cu[s + 1] - cu[s]) + kTB - 1) / kTB;
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int32_t add = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    int32_t run = part[tid] - sum;
    for (int s = s0; s < s1; ++s) {
        tb[s] = run;
        run += (max(0, cu[s + 1] - cu[s]) + kTB - 1) / kTB;
    }
    if (tid == 1023) tb[num_seqs] = part[1023];
}

// Segment and first token of key tile `tile` (tb: tile prefix sums).
__device__ __forceinline__ void tile_origin(const int32_t* cu, const int32_t* tb, int num_seqs,
                                            int tile, int& seg, int& t0, int& rows) {
    seg = find_segment(tb, num_seqs, tile);
    t0 = cu[seg] + kTB * (tile - tb[seg]);
    rows = min(kTB, cu[seg + 1] - t0);
}

// Thread's four 8-value chunks of a 64 x 128 tile: chunk c = tid + 256 i is
// token c / 16, channels 8 (c % 16) + [0, 8); rows >= `rows` read as 0.
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ base, int64_t stride,
                                          int64_t t0, int rows, int head, uint4 (&x)[4]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i;
        const int tok = c >> 4, dc = c & 15;
        x[i] = make_uint4(0, 0, 0, 0);
        if (tok < rows) x[i] = load_stream16(base + (t0 + tok) * stride + head * kD + 8 * dc);
    }
}

// INT8 code of x in a block of maximum magnitude amax: round-half-even of
// 127 x / amax. 127 x is exact for bf16 x and the IEEE division rounds the
// quotient once: an exact half-integer quotient stays exact (and rounds to
// even), any other is at least 2^-16 (relative) from one and stays on its
// side. amax == 0 means every x of the block is 0.
__device__ __forceinline__ int i8_code(float x, float amax) {
    return amax > 0.f ? static_cast<int>(__builtin_rintf((127.0f * x) / amax)) : 0;
}

// INT8 codes of a bf16 chunk (byte j = value j), added to the per-channel
// code sums s[0..7].
__device__ __forceinline__ u32x2 i8_codes8(uint4 raw, float amax, int (&s)[8]) {
    u32x2 out = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int c = i8_code(chunk_val(raw, j), amax);
        s[j] += c;
        out[j >> 2] |= (static_cast<uint32_t>(c) & 0xffu) << (8 * (j & 3));
    }
    return out;
}

// One workgroup per (key tile, head): the codes and block scale of one of
// Q (IS_K false: head-fastest, codes token-major like q, rows past the
// segment end not written) or K (IS_K true: tile-fastest, the 64 x 128 key
// tile, rows past the segment end 0). The K codes of one head are one
// contiguous run of tiles, so tile-fastest workgroups write adjacent 8 KB
// blocks (head-fastest, 7 MB apart at 57,960 tokens, measured 100 against
// 91 us; the transposed V tiles, ordered the same way, gained nothing). I8: INT8 codes (scale amax / 127) instead of
// e4m3, plus the tile's per-channel code sums, int16: qsum [T, H, 128] or
// ksum [H, 16, T, 8] (channel chunk-major).
template <bool I8, bool IS_K>
__global__ __launch_bounds__(256) void quant_qk_kernel(
    const uint16_t* __restrict__ x, int64_t xs, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ tb, int num_seqs, int num_heads, int64_t num_tiles,
    uint8_t* __restrict__ x8, float* __restrict__ xsc, int16_t* __restrict__ xsum) {
    __shared__ float red[4];
    __shared__ int32_t isum[4][I8 ? kD : 1];
    int tile, h;
    if constexpr (IS_K) {   // tile-fastest: consecutive workgroups write adjacent key tiles
        h = static_cast<int>(blockIdx.x / static_cast<unsigned>(num_tiles));
        tile = static_cast<int>(blockIdx.x - static_cast<unsigned>(h) * static_cast<unsigned>(num_tiles));
    } else {
        tile = static_cast<int>(blockIdx.x / static_cast<unsigned>(num_heads));
        h = static_cast<int>(blockIdx.x - static_cast<unsigned>(tile) * num_heads);
    }
    int seg, t0, rows;
    tile_origin(cu, tb, num_seqs, tile, seg, t0, rows);
    const int tid = threadIdx.x, wave = tid >> 6;
    const int64_t row_bytes = static_cast<int64_t>(num_heads) * kD;
    uint4 xv[4];
    load_tile(x, xs, t0, rows, h, xv);
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, absmax8(xv[i]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((tid & 63) == 0) red[wave] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    uint8_t* kt = x8 + ((static_cast<int64_t>(h) * num_tiles + tile) * kTB) * kD;
    const int64_t sidx = static_cast<int64_t>(tile) * num_heads + h;
    if constexpr (I8) {
        // rows past the segment end load as 0, so they add nothing to the sums
        int sm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            const int tok = c >> 4, dc = c & 15;
            const u32x2 cw = i8_codes8(xv[i], amax, sm);
            if constexpr (IS_K)
                __builtin_nontemporal_store(cw, reinterpret_cast<u32x2*>(kt + tok * kD + 8 * dc));
            else if (tok < rows)
                __builtin_nontemporal_store(cw, reinterpret_cast<u32x2*>(x8 + (t0 + tok) * row_bytes + h * kD + 8 * dc));
        }
        // channel chunk tid % 16 is shared with lanes tid ^ 16 and tid ^ 32
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            sm[j] += __shfl_xor(sm[j], 16, 64);
            sm[j] += __shfl_xor(sm[j], 32, 64);
        }
        if ((tid & 63) < 16) {
#pragma unroll
            for (int j = 0; j < 8; ++j) isum[wave][8 * (tid & 15) + j] = sm[j];
        }
        __syncthreads();
        if (tid < kD) {
            const int d = tid;
            const int32_t tot = isum[0][d] + isum[1][d] + isum[2][d] + isum[3][d];
            // |sum| <= 64 * 127 = 8128: int16
            if constexpr (IS_K)   // chunk-major: [H][16 channel chunks][T][8]
                xsum[((static_cast<int64_t>(h) * (kD / 8) + d / 8) * num_tiles + tile) * 8 + d % 8] =
                    static_cast<int16_t>(tot);
            else
                xsum[sidx * kD + d] = static_cast<int16_t>(tot);
        }
        if (tid == 0) xsc[sidx] = amax > 0.f ? amax / 127.0f : 1.0f;
    } else {
        const Fp8Mul mul = fp8_mul_of(amax);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            const int tok = c >> 4, dc = c & 15;
            if constexpr (IS_K)   // K rows past the segment end are 0
                __builtin_nontemporal_store(codes8(xv[i], mul), reinterpret_cast<u32x2*>(kt + tok * kD + 8 * dc));
            else if (tok < rows)
                __builtin_nontemporal_store(codes8(xv[i], mul),
                                            reinterpret_cast<u32x2*>(x8 + (t0 + tok) * row_bytes + h * kD + 8 * dc));
        }
        if (tid == 0) xsc[sidx] = fp8_scale_of(amax);
    }
}

// One workgroup per (key tile, head), head-fastest: the tile's channel amax
// of V, vpart [T, H, 128] (reduced per segment by vscale_kernel). Rows past
// the segment end load as 0 and leave the amax alone.
__global__ __launch_bounds__(256) void vamax_kernel(
    const uint16_t* __restrict__ v, int64_t vs, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ tb, int num_seqs, int num_heads, float* __restrict__ vpart) {
    __shared__ float vred[4][kD];
    const int tile = static_cast<int>(blockIdx.x / static_cast<unsigned>(num_heads));
    const int h = static_cast<int>(blockIdx.x - static_cast<unsigned>(tile) * num_heads);
    int seg, t0, rows;
    tile_origin(cu, tb, num_seqs, tile, seg, t0, rows);
    const int tid = threadIdx.x, wave = tid >> 6;
    uint4 xv[4];
    load_tile(v, vs, t0, rows, h, xv);
    // the 4 tokens tid / 16 + 16 i share channel chunk tid % 16 with lanes
    // tid ^ 16 and tid ^ 32
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float a = fmaxf(fmaxf(fabsf(chunk_val(xv[0], j)), fabsf(chunk_val(xv[1], j))),
                        fmaxf(fabsf(chunk_val(xv[2], j)), fabsf(chunk_val(xv[3], j))));
        a = fmaxf(a, __shfl_xor(a, 16, 64));
        a = fmaxf(a, __shfl_xor(a, 32, 64));
        if ((tid & 63) < 16) vred[wave][8 * (tid & 15) + j] = a;
    }
    __syncthreads();
    if (tid < kD) {
        const float a = fmaxf(fmaxf(vred[0][tid], vred[1][tid]), fmaxf(vred[2][tid], vred[3][tid]));
        vpart[(static_cast<int64_t>(tile) * num_heads + h) * kD + tid] = a;
    }
}

// v_scale[s, h, c] (and the channel amax) from the tile partials of segment s. Block: 32 columns x
// 32 tile slices, eight loads in flight per thread; grid (B, H * 128 / 32).
__global__ __launch_bounds__(1024) void vscale_kernel(const float* __restrict__ vpart,
                                                      const int32_t* __restrict__ tb, int num_heads,
                                                      float* __restrict__ vsc, float* __restrict__ vamax) {
    __shared__ float red[32][33];
    const int seg = blockIdx.x;
    const int col = threadIdx.x & 31, slice = threadIdx.x >> 5;
    const int64_t cols = static_cast<int64_t>(num_heads) * kD;
    const int64_t c = static_cast<int64_t>(blockIdx.y) * 32 + col;
    const int end = tb[seg + 1];
    float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int j = tb[seg] + slice;
    for (; j + 7 * 32 < end; j += 8 * 32) {
#pragma unroll
        for (int u = 0; u < 8; ++u) m[u] = fmaxf(m[u], vpart[(j + 32 * u) * cols + c]);
    }
    for (; j < end; j += 32) m[0] = fmaxf(m[0], vpart[j * cols + c]);
    float mm = fmaxf(fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3])), fmaxf(fmaxf(m[4], m[5]), fmaxf(m[6], m[7])));
    red[slice][col] = mm;
    __syncthreads();
    if (slice == 0) {
        for (int i = 1; i < 32; ++i) mm = fmaxf(mm, red[i][col]);
        vsc[seg * cols + c] = fp8_scale_of(mm);
        vamax[seg * cols + c] = mm;
    }
}

// One wave per (key tile, head), head-fastest, four waves per workgroup
// (single-wave workgroups measured 1.6 % slower over the whole quantise
// pass): V codes of the tile, transposed and key-permuted, straight to HBM. Lane 16 u + dc (u = 2 b + g)
// owns the 16-byte chunk 2 g + b (positions 16 (2 g + b) .. + 15) of channel
// rows 8 dc .. 8 dc + 7; those positions hold keys 32 b + 8 i + 4 g + e
// (i, e in 0..3, position 16 (2 g + b) + 4 i + e), so the lane reads channels
// 8 dc .. 8 dc + 7 of those 16 keys and writes eight 16-byte chunks.
__global__ __launch_bounds__(256) void quant_v_kernel(
    const uint16_t* __restrict__ v, int64_t vs, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ tb, int num_seqs, int num_heads, int64_t num_tiles,
    const float* __restrict__ vamax, uint8_t* __restrict__ v8t, unsigned items) {
    const unsigned item = blockIdx.x * 4u + (threadIdx.x >> 6);
    if (item >= items) return;
    const int tile = static_cast<int>(item / static_cast<unsigned>(num_heads));
    const int h = static_cast<int>(item - static_cast<unsigned>(tile) * num_heads);
    int seg, t0, rows;
    tile_origin(cu, tb, num_seqs, tile, seg, t0, rows);
    const int lane = threadIdx.x & 63, dc = lane & 15, u = lane >> 4, g = u & 1, b = u >> 1;
    uint4 x[16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int key = 32 * b + 8 * i + 4 * g + e;
            x[4 * i + e] = make_uint4(0, 0, 0, 0);
            if (key < rows) x[4 * i + e] = load_stream16(v + (t0 + key) * vs + h * kD + 8 * dc);
        }
    const float4* am4 = reinterpret_cast<const float4*>(vamax + (static_cast<int64_t>(seg) * num_heads + h) * kD + 8 * dc);
    const float4 a0 = am4[0], a1 = am4[1];
    const float am[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    uint8_t* dst = v8t + ((static_cast<int64_t>(h) * num_tiles + tile) * kD + 8 * dc) * kTB + 16 * (2 * g + b);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const Fp8Mul m = fp8_mul_of(am[j]);
        uint4 w;
        uint32_t* wp = reinterpret_cast<uint32_t*>(&w);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t c = e4m3x2<false>(fp8_prep(chunk_val(x[4 * i], j), m),
                                             fp8_prep(chunk_val(x[4 * i + 1], j), m), 0u);
            wp[i] = e4m3x2<true>(fp8_prep(chunk_val(x[4 * i + 2], j), m),
                                 fp8_prep(chunk_val(x[4 * i + 3], j), m), c);
        }
        *reinterpret_cast<uint4*>(dst + j * kTB) = w;   // plain: L2 joins the 64-byte halves of each line
    }
}

}  // namespace

size_t fp8_tiles_upper_bound(int num_seqs, int total_tokens) {
    return (static_cast<size_t>(total_tokens) + static_cast<size_t>(num_seqs) * (kTB - 1)) / kTB;
}

// Workspace: tb int32[B + 1] | vamax float[B, H, 128] | vpart float[T, H, 128].
size_t fp8_quant_workspace_bytes(int num_seqs, int total_tokens, int num_heads) {
    const size_t t = fp8_tiles_upper_bound(num_seqs, total_tokens);
    const size_t tb = ((static_cast<size_t>(num_seqs) + 1) * sizeof(int32_t) + 255) & ~size_t(255);
    const size_t va = (static_cast<size_t>(num_seqs) * num_heads * kD * sizeof(float) + 255) & ~size_t(255);
    return tb + va + t * num_heads * kD * sizeof(float);
}

hipError_t launch_fp8_quantize(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t qs,
                               int64_t ks, int64_t vs, const int32_t* cu, int num_seqs,
                               int num_heads, int64_t num_tiles, uint8_t* q8, uint8_t* k8,
                               uint8_t* v8t, float* qsc, float* ksc, float* vsc, void* workspace,
                               hipStream_t stream, int16_t* qsum, int16_t* ksum) {
    if (num_seqs <= 0 || num_tiles <= 0) return hipSuccess;
    if (num_tiles * num_heads > 0xffffffffll) return hipErrorInvalidValue;   // 1-D grid of (tile, head)
    int32_t* tb = static_cast<int32_t*>(workspace);
    const size_t tb_bytes = ((static_cast<size_t>(num_seqs) + 1) * sizeof(int32_t) + 255) & ~size_t(255);
    const size_t va_bytes = (static_cast<size_t>(num_seqs) * num_heads * kD * sizeof(float) + 255) & ~size_t(255);
    float* vamax = reinterpret_cast<float*>(static_cast<char*>(workspace) + tb_bytes);
    float* vpart = reinterpret_cast<float*>(static_cast<char*>(workspace) + tb_bytes + va_bytes);
    hipLaunchKernelGGL(tile64_scan_kernel, dim3(1), dim3(1024), 0, stream, cu, num_seqs, tb);
    const unsigned items = static_cast<unsigned>(num_tiles * num_heads);
    if (qsum != nullptr) {
        hipLaunchKernelGGL((quant_qk_kernel<true, false>), dim3(items), dim3(256), 0, stream, q, qs, cu, tb,
                           num_seqs, num_heads, num_tiles, q8, qsc, qsum);
        hipLaunchKernelGGL((quant_qk_kernel<true, true>), dim3(items), dim3(256), 0, stream, k, ks, cu, tb,
                           num_seqs, num_heads, num_tiles, k8, ksc, ksum);
    } else {
        hipLaunchKernelGGL((quant_qk_kernel<false, false>), dim3(items), dim3(256), 0, stream, q, qs, cu, tb,
                           num_seqs, num_heads, num_tiles, q8, qsc, nullptr);
        hipLaunchKernelGGL((quant_qk_kernel<false, true>), dim3(items), dim3(256), 0, stream, k, ks, cu, tb,
                           num_seqs, num_heads, num_tiles, k8, ksc, nullptr);
    }
    hipLaunchKernelGGL(vamax_kernel, dim3(items), dim3(256), 0, stream, v, vs, cu, tb, num_seqs, num_heads,
                       vpart);
    hipLaunchKernelGGL(vscale_kernel, dim3(num_seqs, num_heads * kD / 32), dim3(1024), 0, stream,
                       vpart, tb, num_heads, vsc, vamax);
    hipLaunchKernelGGL(quant_v_kernel, dim3((items + 3) / 4), dim3(256), 0, stream, v, vs, cu, tb, num_seqs,
                       num_heads, num_tiles, vamax, v8t, items);
    return hipGetLastError();
}

}  // namespace h3
