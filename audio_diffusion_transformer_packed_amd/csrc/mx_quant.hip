// MXFP8 quantisation of bf16 rows, for the block linears' weights (once, at
// load time) and for activations that reach a linear from a kernel without
// a fused quantiser (the attention output). "MiniMax H3 on Ascend 950PR /
// 950DT", section "Recommended lossy configuration": the transformer runs
// with MXFP8 online quantization. The format is the OCP MX v1.0 one (the
// pages do not give it): per row, blocks of 32 consecutive elements share an
// E8M0 scale 2^(floor(log2 amax) - 8) (never below 2^-127) and each element
// is E4M3(x / scale), round to nearest even, saturating at +-448.
//
// Layouts: codes [rows, k] row-major (one byte per element); scales K-step-
// major, the scale of row r and block j at byte ((j / 4) rows + r) 4 + j % 4.
// For bf16 x every step is exact in fp32 (amax, the power-of-two scaling),
// so the codes equal the definition bit for bit.
//
// MXFP4 ("MiniMax H3 on Ascend 950PR / 950DT", section "MXFP4 online
// quantization", OCP MX v1.0 MXFP4): scale 2^(floor(log2 amax) - 2) and
// E2M1 elements (nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, midpoints to the
// even index, saturating at 6; sign bit 3 from the input), two per byte
// (codes [rows, k / 2], element 2i in the low nibble of byte i); scales
// 8 bytes per row and 256-element K step, the step's even blocks in the
// first dword and its odd blocks in the second (the order in which the
// matrix core's lanes take them).
#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {
namespace {

constexpr int kChunksPerThread = 4;   // 16-byte loads in flight per thread

// One lane per 8-element chunk (16-byte load), four consecutive lanes per
// block; each thread takes four chunks 256 apart and issues all four loads
// before converting any (one load per thread at a time, grid-stride,
// measured 100 against 91 us at 57,960 x 3072; eight per thread 91 us).
// k % 32 == 0, so a block's four lanes always agree on whether a chunk
// exists and the row's chunk count is a multiple of 4.
__global__ __launch_bounds__(256) void mx_quant_kernel(const uint16_t* __restrict__ x, int64_t ld,
                                                       int64_t rows, int64_t k,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
    const int64_t per_row = k >> 3;
    const int64_t nchunk = rows * per_row;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * (kChunksPerThread * 256) + threadIdx.x;
    uint4 raws[kChunksPerThread];
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
        const int64_t c = c0 + 256 * u;
        if (c < nchunk) {
            const int64_t r = c / per_row, ch = c - r * per_row;
            raws[u] = load_stream16(x + r * ld + ch * 8);
        }
    }
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
        const int64_t c = c0 + 256 * u;
        if (c >= nchunk) break;   // a block's four lanes share c / 4
        const int64_t r = c / per_row, ch = c - r * per_row;
        const uint32_t w[4] = {raws[u].x, raws[u].y, raws[u].z, raws[u].w};
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
        float am = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
        am = fmaxf(am, __shfl_xor(am, 1, 64));
        am = fmaxf(am, __shfl_xor(am, 2, 64));
        const uint32_t sb = mx_scale_byte(am);
        const float inv = mx_inv_scale(sb);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= inv;
        *reinterpret_cast<uint2*>(codes + r * k + ch * 8) = mx_codes8(v);
        if ((ch & 3) == 0) scales[mx_scale_offset(r, ch >> 2, rows)] = static_cast<uint8_t>(sb);
    }
}

// MXFP4: the same lane layout; a lane's 8 elements become one dword of
// codes (element 2i in the low nibble of byte i), rounded by the hardware
// fp4 conversion (e2m1x8; a chain of seven compares per element instead
// measured 137 against 83 us at 57,960 x 3072, with one load per thread at
// a time; four in flight: 78 us).
__global__ __launch_bounds__(256) void mx4_quant_kernel(const uint16_t* __restrict__ x, int64_t ld,
                                                        int64_t rows, int64_t k,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales) {
    const int64_t per_row = k >> 3;
    const int64_t nchunk = rows * per_row;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * (kChunksPerThread * 256) + threadIdx.x;
    uint4 raws[kChunksPerThread];
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
        const int64_t c = c0 + 256 * u;
        if (c < nchunk) {
            const int64_t r = c / per_row, ch = c - r * per_row;
            raws[u] = load_stream16(x + r * ld + ch * 8);
        }
    }
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
        const int64_t c = c0 + 256 * u;
        if (c >= nchunk) break;   // a block's four lanes share c / 4
        const int64_t r = c / per_row, ch = c - r * per_row;
        const uint32_t w[4] = {raws[u].x, raws[u].y, raws[u].z, raws[u].w};
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
        float am = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
        am = fmaxf(am, __shfl_xor(am, 1, 64));
        am = fmaxf(am, __shfl_xor(am, 2, 64));
        const uint32_t sb = mx4_scale_byte(am);
        const float inv = mx_inv_scale(sb);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= inv;
        *reinterpret_cast<uint32_t*>(codes + r * (k >> 1) + ch * 4) = e2m1x8(v);
        if ((ch & 3) == 0) scales[mx4_scale_offset(r, ch >> 2, rows)] = static_cast<uint8_t>(sb);
    }
}

}  // namespace

hipError_t launch_mx4_quantize(const uint16_t* x, int64_t ld, int64_t rows, int64_t k, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const int64_t nchunk = rows * (k / 8);
    const int64_t blocks = (nchunk + kChunksPerThread * 256 - 1) / (kChunksPerThread * 256);
    if (blocks > 0xffffffffll) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mx4_quant_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, x, ld,
                       rows, k, codes, scales);
    return hipGetLastError();
}

hipError_t launch_mx_quantize(const uint16_t* x, int64_t ld, int64_t rows, int64_t k, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const int64_t nchunk = rows * (k / 8);
    const int64_t blocks = (nchunk + kChunksPerThread * 256 - 1) / (kChunksPerThread * 256);
    if (blocks > 0xffffffffll) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mx_quant_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, x, ld,
                       rows, k, codes, scales);
    return hipGetLastError();
}

}  // namespace h3
