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
// For bf16 x, 448 x is exact in fp32 and one IEEE division decides exactly
// (a quotient on a rounding midpoint stays on it and goes to the even code;
// any other is far from one), so no rounded scale enters the decision.
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
// All HBM-bound; each kernel reads its input once with 16-byte loads.
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

// Divisor of 448 x for the code (amax, or 1 when amax == 0 and x == 0).
__device__ __forceinline__ float fp8_den_of(float amax) { return amax > 0.f ? amax : 1.0f; }

// Two fp32 -> two e4m3 codes in the low 16 bits.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
    a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
    b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xffffu;
}

// Codes of x[j0 .. j0+3]: RNE(448 x / den), four bytes.
__device__ __forceinline__ uint32_t codes4(const float (&x)[8], int j0, float den) {
    return e4m3x2(kE4M3Max * x[j0] / den, kE4M3Max * x[j0 + 1] / den) |
           (e4m3x2(kE4M3Max * x[j0 + 2] / den, kE4M3Max * x[j0 + 3] / den) << 16);
}

__device__ __forceinline__ float block_max(float v, float* red) {
    v = fmaxf(v, __shfl_xor(v, 32, 64));
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    v = fmaxf(v, __shfl_xor(v, 8, 64));
    v = fmaxf(v, __shfl_xor(v, 4, 64));
    v = fmaxf(v, __shfl_xor(v, 2, 64));
    v = fmaxf(v, __shfl_xor(v, 1, 64));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return m;
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
                                          int64_t t0, int rows, int head, float (&x)[4][8]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i;
        const int tok = c >> 4, dc = c & 15;
        u32x4 raw = {0, 0, 0, 0};
        if (tok < rows)
            raw = *reinterpret_cast<const u32x4*>(base + (t0 + tok) * stride + head * kD + 8 * dc);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[i][2 * j] = __uint_as_float(raw[j] << 16);
            x[i][2 * j + 1] = __uint_as_float(raw[j] & 0xffff0000u);
        }
    }
}

// One workgroup per (key tile, head): Q and K codes + block scales, and the
// tile's channel amax of V (reduced per segment afterwards).
__global__ __launch_bounds__(256) void quant_qk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int64_t qs, int64_t ks, int64_t vs, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ tb, int num_seqs, int num_heads, int64_t num_tiles,
    uint8_t* __restrict__ q8, uint8_t* __restrict__ k8, float* __restrict__ qsc,
    float* __restrict__ ksc, float* __restrict__ vpart) {
    __shared__ float red[4];
    __shared__ float vred[4][kD];
    const int tile = blockIdx.x, h = blockIdx.y;
    int seg, t0, rows;
    tile_origin(cu, tb, num_seqs, tile, seg, t0, rows);
    const int tid = threadIdx.x;
    const int64_t row_bytes = static_cast<int64_t>(num_heads) * kD;
    float xq[4][8], xk[4][8], xv[4][8];
    load_tile(q, qs, t0, rows, h, xq);
    load_tile(k, ks, t0, rows, h, xk);
    load_tile(v, vs, t0, rows, h, xv);
    float mq = 0.f, mk = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            mq = fmaxf(mq, fabsf(xq[i][j]));
            mk = fmaxf(mk, fabsf(xk[i][j]));
        }
    const float amax_q = block_max(mq, red);
    const float amax_k = block_max(mk, red);
    const float dq = fp8_den_of(amax_q), dk = fp8_den_of(amax_k);
    uint8_t* kt = k8 + ((static_cast<int64_t>(h) * num_tiles + tile) * kTB) * kD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i;
        const int tok = c >> 4, dc = c & 15;
        if (tok < rows) {
            u32x2 w;
            w.x = codes4(xq[i], 0, dq);
            w.y = codes4(xq[i], 4, dq);
            *reinterpret_cast<u32x2*>(q8 + (t0 + tok) * row_bytes + h * kD + 8 * dc) = w;
        }
        u32x2 w;                              // K rows past the segment end are 0
        w.x = codes4(xk[i], 0, dk);
        w.y = codes4(xk[i], 4, dk);
        *reinterpret_cast<u32x2*>(kt + tok * kD + 8 * dc) = w;
    }
    if (tid == 0) {
        qsc[static_cast<int64_t>(tile) * num_heads + h] = fp8_scale_of(amax_q);
        ksc[static_cast<int64_t>(tile) * num_heads + h] = fp8_scale_of(amax_k);
    }
    // V: channel amax over this tile's tokens; the 4 tokens tid / 16 + 16 i
    // share channel chunk tid % 16 with lanes tid ^ 16 and tid ^ 32
    float vm[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float a = fmaxf(fmaxf(fabsf(xv[0][j]), fabsf(xv[1][j])), fmaxf(fabsf(xv[2][j]), fabsf(xv[3][j])));
        a = fmaxf(a, __shfl_xor(a, 16, 64));
        a = fmaxf(a, __shfl_xor(a, 32, 64));
        vm[j] = a;
    }
    if ((tid & 63) < 16) {
#pragma unroll
        for (int j = 0; j < 8; ++j) vred[tid >> 6][8 * (tid & 15) + j] = vm[j];
    }
    __syncthreads();
    if (tid < kD) {
        const float a = fmaxf(fmaxf(vred[0][tid], vred[1][tid]), fmaxf(vred[2][tid], vred[3][tid]));
        vpart[(static_cast<int64_t>(tile) * num_heads + h) * kD + tid] = a;
    }
}

// v_scale[s, h, c] (and the channel amax) from the tile partials of segment s. Block: 32 columns x
// 32 tile slices; grid (B, H * 128 / 32).
__global__ __launch_bounds__(1024) void vscale_kernel(const float* __restrict__ vpart,
                                                      const int32_t* __restrict__ tb, int num_heads,
                                                      float* __restrict__ vsc, float* __restrict__ vamax) {
    __shared__ float red[32][33];
    const int seg = blockIdx.x;
    const int col = threadIdx.x & 31, slice = threadIdx.x >> 5;
    const int64_t cols = static_cast<int64_t>(num_heads) * kD;
    const int64_t c = static_cast<int64_t>(blockIdx.y) * 32 + col;
    float m = 0.f;
    for (int j = tb[seg] + slice; j < tb[seg + 1]; j += 32) m = fmaxf(m, vpart[j * cols + c]);
    red[slice][col] = m;
    __syncthreads();
    if (slice == 0) {
        for (int i = 1; i < 32; ++i) m = fmaxf(m, red[i][col]);
        vsc[seg * cols + c] = fp8_scale_of(m);
        vamax[seg * cols + c] = m;
    }
}

// One workgroup per (key tile, head): V codes, transposed and permuted
// through LDS, written as one contiguous 8 KB block.
__global__ __launch_bounds__(256) void quant_v_kernel(
    const uint16_t* __restrict__ v, int64_t vs, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ tb, int num_seqs, int num_heads, int64_t num_tiles,
    const float* __restrict__ vamax, uint8_t* __restrict__ v8t) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kD * kTB];
    const int tile = blockIdx.x, h = blockIdx.y;
    int seg, t0, rows;
    tile_origin(cu, tb, num_seqs, tile, seg, t0, rows);
    const int tid = threadIdx.x;
    float x[4][8];
    load_tile(v, vs, t0, rows, h, x);
    const int dc = tid & 15;
    float den[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        den[j] = fp8_den_of(vamax[(static_cast<int64_t>(seg) * num_heads + h) * kD + 8 * dc + j]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int key = (tid >> 4) + 16 * i;
        const int b = key >> 5, r = key & 31;
        const int pos = 32 * ((r >> 2) & 1) + 16 * b + 4 * (r >> 3) + (r & 3);
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            const uint32_t w = e4m3x2(kE4M3Max * x[i][j] / den[j], kE4M3Max * x[i][j + 1] / den[j + 1]);
            lds[(8 * dc + j) * kTB + pos] = static_cast<uint8_t>(w & 0xff);
            lds[(8 * dc + j + 1) * kTB + pos] = static_cast<uint8_t>(w >> 8);
        }
    }
    __syncthreads();
    uint8_t* dst = v8t + ((static_cast<int64_t>(h) * num_tiles + tile) * kD) * kTB;
    const u32x4* src = reinterpret_cast<const u32x4*>(lds);
    reinterpret_cast<u32x4*>(dst)[tid] = src[tid];
    reinterpret_cast<u32x4*>(dst)[tid + 256] = src[tid + 256];
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
                               hipStream_t stream) {
    if (num_seqs <= 0 || num_tiles <= 0) return hipSuccess;
    int32_t* tb = static_cast<int32_t*>(workspace);
    const size_t tb_bytes = ((static_cast<size_t>(num_seqs) + 1) * sizeof(int32_t) + 255) & ~size_t(255);
    const size_t va_bytes = (static_cast<size_t>(num_seqs) * num_heads * kD * sizeof(float) + 255) & ~size_t(255);
    float* vamax = reinterpret_cast<float*>(static_cast<char*>(workspace) + tb_bytes);
    float* vpart = reinterpret_cast<float*>(static_cast<char*>(workspace) + tb_bytes + va_bytes);
    hipLaunchKernelGGL(tile64_scan_kernel, dim3(1), dim3(1024), 0, stream, cu, num_seqs, tb);
    hipLaunchKernelGGL(quant_qk_kernel, dim3(static_cast<unsigned>(num_tiles), num_heads), dim3(256), 0, stream,
                       q, k, v, qs, ks, vs, cu, tb, num_seqs, num_heads, num_tiles, q8, k8, qsc, ksc,
                       vpart);
    hipLaunchKernelGGL(vscale_kernel, dim3(num_seqs, num_heads * kD / 32), dim3(1024), 0, stream,
                       vpart, tb, num_heads, vsc, vamax);
    hipLaunchKernelGGL(quant_v_kernel, dim3(static_cast<unsigned>(num_tiles), num_heads), dim3(256), 0,
                       stream, v, vs, cu, tb, num_seqs, num_heads, num_tiles, vamax, v8t);
    return hipGetLastError();
}

}  // namespace h3
