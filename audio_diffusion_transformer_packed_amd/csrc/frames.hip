// Decoded frames to contiguous uint8: FP32 [B, C, T, H, W] -> uint8 [B, T, H,
// W, C] ("FastH3 在八卡 B300 上实现完整 MP4 生成快于播放时长", section
// "紧凑输出与并行 MP4 构建"; "MiniMax H3 FastH3 real-time serving with
// vLLM-Omni", section "System-wide optimizations in vLLM-Omni", GPU output
// preparation bullet: converted once on the GPU, a quarter of the bytes).
// Value map (the pages give none; the decoded-video convention for [-1, 1]):
//   u = round_half_even(255 * clamp(x / 2 + 1/2, 0, 1)), NaN -> 0,
// the exact value for the fp32 input (no intermediate rounding decides a
// level). For x in (-1, 1), y = 127.5 + 127.5 x: the product is exact in
// fp64 and one fma rounds the sum once. Writing x = M 2^E (M of 24 bits),
// y - (k + 1/2) = (255 x + 254 - 2k) / 2 is a nonzero multiple of 2^(E-1)
// unless x = 0, so for |x| >= 2^-20 (E >= -43) y stays at least 2^-44 from
// every midpoint, more than the fma's rounding (<= 2^-46 below 256) can
// cross, and rint of the fp64 value is the exact level. For |x| < 2^-20 the
// level is 127 for negative x and 128 otherwise (x = 0 is the tie 127.5,
// which goes to the even 128). An fp32 evaluation of x * 0.5 + 0.5 would
// instead send every negative x above -2^-25 to 128 and misplace 674 other
// fp32 inputs next to midpoints.
//
// HBM-bound (4 C bytes read and C written per pixel). Vector path: a wave
// takes 1024 consecutive pixels, reads them with 1 KB-contiguous 16-byte
// nontemporal loads per channel plane, interleaves the channels in LDS and
// writes 1 KB-contiguous 16-byte stores. Otherwise (T H W not a multiple of
// 16, C > 4 or unaligned buffers) one thread per pixel.
#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {
namespace {

__device__ __forceinline__ uint32_t to_u8(float x) {
    double y = __builtin_fma(127.5, static_cast<double>(x), 127.5);
    y = __builtin_fmin(__builtin_fmax(y, 0.0), 255.0);   // in range for the conversion
    uint32_t u = static_cast<uint32_t>(__builtin_rint(y));
    u = __builtin_fabsf(x) < 0x1p-20f ? (x < 0.0f ? 127u : 128u) : u;
    u = x >= 1.0f ? 255u : u;
    return x > -1.0f ? u : 0u;              // x <= -1, -inf and NaN give 0
}

// One wave per 1024 consecutive pixels of one batch entry: load q (0..3) of
// lane i reads pixels 256 q + 4 i .. + 3 of every channel plane (each load
// instruction covers 1 KB contiguous), the wave assembles its 1024 C output
// bytes in LDS (lane i, load q: 4 C bytes at C (256 q + 4 i), C dword writes,
// conflict-free) and stores them as C contiguous 1 KB runs. Pixels past the
// end (only in a frame sequence's last wave) load as 0 and are not stored.
template <int C>
__global__ __launch_bounds__(256) void frames_u8_vec_kernel(const float* __restrict__ x,
                                                           uint8_t* __restrict__ out, int64_t waves,
                                                           int64_t waves_per_b, int64_t pixels) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[4][1024 * C];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (gw >= waves) return;                       // whole wave: no barrier below
    const int64_t b = gw / waves_per_b;
    const int64_t p_base = (gw - b * waves_per_b) * 1024;
    uint8_t* l = lds[wave];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t p = p_base + 256 * q + 4 * lane;
        uint32_t v[C][4];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            uint4 raw = make_uint4(0, 0, 0, 0);
            if (p < pixels) raw = load_stream16(x + (b * C + c) * pixels + p);
            v[c][0] = to_u8(__uint_as_float(raw.x));
            v[c][1] = to_u8(__uint_as_float(raw.y));
            v[c][2] = to_u8(__uint_as_float(raw.z));
            v[c][3] = to_u8(__uint_as_float(raw.w));
        }
        // bytes k = 0 .. 4C-1 of these 4 pixels: pixel k / C, channel k % C
#pragma unroll
        for (int d = 0; d < C; ++d) {
            uint32_t word = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = 4 * d + j;
                word |= v[k % C][k / C] << (8 * j);
            }
            *reinterpret_cast<uint32_t*>(l + C * (256 * q + 4 * lane) + 4 * d) = word;
        }
    }
    // the wave's own LDS bytes only: its LDS operations complete in order
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int64_t obytes = (pixels - p_base) * C;  // bytes of this sequence left from p_base
    uint8_t* dst = out + (b * pixels + p_base) * C;
#pragma unroll
    for (int s = 0; s < C; ++s) {
        const int off = 1024 * s + 16 * lane;
        if (off < obytes) store_stream16(dst + off, *reinterpret_cast<const uint4*>(l + off));
    }
}

__global__ __launch_bounds__(256) void frames_u8_pixel_kernel(const float* __restrict__ x,
                                                             uint8_t* __restrict__ out, int64_t b_count,
                                                             int c_count, int64_t pixels) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= b_count * pixels) return;
    const int64_t b = gid / pixels, p = gid - b * pixels;
    for (int c = 0; c < c_count; ++c)
        out[gid * c_count + c] = static_cast<uint8_t>(to_u8(x[(b * c_count + c) * pixels + p]));
}

}  // namespace

hipError_t launch_frames_to_u8(const float* x, uint8_t* out, int64_t b, int c, int64_t pixels,
                               hipStream_t stream) {
    if (b == 0 || c == 0 || pixels == 0) return hipSuccess;
    const bool aligned = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
    if (aligned && pixels % 16 == 0 && c <= 4) {
        const int64_t wpb = (pixels + 1023) / 1024, waves = b * wpb;
        const dim3 grid(static_cast<unsigned>((waves + 3) / 4));
        switch (c) {
            case 1: hipLaunchKernelGGL(frames_u8_vec_kernel<1>, grid, dim3(256), 0, stream, x, out, waves, wpb, pixels); break;
            case 2: hipLaunchKernelGGL(frames_u8_vec_kernel<2>, grid, dim3(256), 0, stream, x, out, waves, wpb, pixels); break;
            case 3: hipLaunchKernelGGL(frames_u8_vec_kernel<3>, grid, dim3(256), 0, stream, x, out, waves, wpb, pixels); break;
            default: hipLaunchKernelGGL(frames_u8_vec_kernel<4>, grid, dim3(256), 0, stream, x, out, waves, wpb, pixels); break;
        }
    } else {
        const dim3 grid(static_cast<unsigned>((b * pixels + 255) / 256));
        hipLaunchKernelGGL(frames_u8_pixel_kernel, grid, dim3(256), 0, stream, x, out, b, c, pixels);
    }
    return hipGetLastError();
}

}  // namespace h3
