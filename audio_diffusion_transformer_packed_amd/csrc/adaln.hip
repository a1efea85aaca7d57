// AdaLN for the packed sequence ("MiniMax H3 FastH3 real-time serving with
// vLLM-Omni", section "System-wide optimizations in vLLM-Omni", fused DiT
// operators bullet: modulation and normalization fused).
//
//  * modulation GEMV: mod[b, :] = cond[b, :] . W_mod^T in fp32; HBM-bound on
//    the 6C x C weight, one wave per weight row, every segment's cond is
//    applied to the row while it is in registers;
//  * RMSNorm + modulate: h[t] = RMSNorm(x[t]) * (1 + scale[seg(t)]) +
//    shift[seg(t)]; one wave per token row, 16-byte coalesced loads, the
//    row's sum of squares reduced across the wave, one bf16 rounding.
#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {
namespace {

constexpr int kThreads = 256;

template <int NCH>
__global__ __launch_bounds__(kThreads) void modulation_kernel(
    const uint16_t* __restrict__ cond, const uint16_t* __restrict__ w, float* __restrict__ mod,
    int num_seqs, int hidden, int rows) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (row >= rows) return;
    float wr[NCH * 8];
    const uint16_t* wp = w + static_cast<int64_t>(row) * hidden;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        Chunk16 c;
        c.u = *reinterpret_cast<const uint4*>(wp + (i * 64 + lane) * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) wr[i * 8 + e] = bf2f(c.h[e]);
    }
    for (int b = 0; b < num_seqs; ++b) {
        const uint16_t* cp = cond + static_cast<int64_t>(b) * hidden;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            Chunk16 c;
            c.u = *reinterpret_cast<const uint4*>(cp + (i * 64 + lane) * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf(bf2f(c.h[e]), wr[i * 8 + e], acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) mod[static_cast<int64_t>(b) * rows + row] = acc;
    }
}

template <int NCH>
__global__ __launch_bounds__(kThreads) void adaln_kernel(
    const uint16_t* __restrict__ x, uint16_t* __restrict__ h, const float* __restrict__ shift,
    const float* __restrict__ scale, int64_t mod_stride, const int32_t* __restrict__ cu,
    int num_seqs, int total_tokens, int hidden, float eps) {
    const int lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
    if (t >= total_tokens) return;
    const int seg = num_seqs == 1 ? 0 : find_segment(cu, num_seqs, t);
    const uint16_t* xp = x + t * hidden;
    Chunk16 xc[NCH];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        xc[i].u = *reinterpret_cast<const uint4*>(xp + (i * 64 + lane) * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float f = bf2f(xc[i].h[e]);
            ss = fmaf(f, f, ss);
        }
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(fmaf(ss, 1.0f / hidden, eps));
    const float* shp = shift + static_cast<int64_t>(seg) * mod_stride;
    const float* scp = scale + static_cast<int64_t>(seg) * mod_stride;
    uint16_t* hp = h + t * hidden;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c0 = (i * 64 + lane) * 8;
        const float4 sh0 = *reinterpret_cast<const float4*>(shp + c0);
        const float4 sh1 = *reinterpret_cast<const float4*>(shp + c0 + 4);
        const float4 sc0 = *reinterpret_cast<const float4*>(scp + c0);
        const float4 sc1 = *reinterpret_cast<const float4*>(scp + c0 + 4);
        const float shv[8] = {sh0.x, sh0.y, sh0.z, sh0.w, sh1.x, sh1.y, sh1.z, sh1.w};
        const float scv[8] = {sc0.x, sc0.y, sc0.z, sc0.w, sc1.x, sc1.y, sc1.z, sc1.w};
        Chunk16 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = fmaf(bf2f(xc[i].h[2 * e]) * r, 1.0f + scv[2 * e], shv[2 * e]);
            const float b = fmaf(bf2f(xc[i].h[2 * e + 1]) * r, 1.0f + scv[2 * e + 1], shv[2 * e + 1]);
            out.w[e] = pack_bf16x2(a, b);
        }
        *reinterpret_cast<uint4*>(hp + c0) = out.u;
    }
}

#define H3_NCH_CASE(N, KERNEL)                                                               \
    case N:                                                                                  \
        hipLaunchKernelGGL(KERNEL<N>, grid, dim3(kThreads), 0, stream, args...);             \
        break;

template <typename... Args>
hipError_t launch_modulation_nch(int nch, dim3 grid, hipStream_t stream, Args... args) {
    switch (nch) {
        H3_NCH_CASE(1, modulation_kernel) H3_NCH_CASE(2, modulation_kernel)
        H3_NCH_CASE(3, modulation_kernel) H3_NCH_CASE(4, modulation_kernel)
        H3_NCH_CASE(5, modulation_kernel) H3_NCH_CASE(6, modulation_kernel)
        H3_NCH_CASE(7, modulation_kernel) H3_NCH_CASE(8, modulation_kernel)
        H3_NCH_CASE(9, modulation_kernel) H3_NCH_CASE(10, modulation_kernel)
        H3_NCH_CASE(11, modulation_kernel) H3_NCH_CASE(12, modulation_kernel)
        H3_NCH_CASE(13, modulation_kernel) H3_NCH_CASE(14, modulation_kernel)
        H3_NCH_CASE(15, modulation_kernel) H3_NCH_CASE(16, modulation_kernel)
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename... Args>
hipError_t launch_adaln_nch(int nch, dim3 grid, hipStream_t stream, Args... args) {
    switch (nch) {
        H3_NCH_CASE(1, adaln_kernel) H3_NCH_CASE(2, adaln_kernel)
        H3_NCH_CASE(3, adaln_kernel) H3_NCH_CASE(4, adaln_kernel)
        H3_NCH_CASE(5, adaln_kernel) H3_NCH_CASE(6, adaln_kernel)
        H3_NCH_CASE(7, adaln_kernel) H3_NCH_CASE(8, adaln_kernel)
        H3_NCH_CASE(9, adaln_kernel) H3_NCH_CASE(10, adaln_kernel)
        H3_NCH_CASE(11, adaln_kernel) H3_NCH_CASE(12, adaln_kernel)
        H3_NCH_CASE(13, adaln_kernel) H3_NCH_CASE(14, adaln_kernel)
        H3_NCH_CASE(15, adaln_kernel) H3_NCH_CASE(16, adaln_kernel)
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
#undef H3_NCH_CASE

}  // namespace

hipError_t launch_modulation(const uint16_t* cond, const uint16_t* w_mod, float* mod,
                             int num_seqs, int hidden, hipStream_t stream) {
    if (num_seqs == 0) return hipSuccess;
    const int rows = 6 * hidden;
    const dim3 grid((rows + 3) / 4);
    return launch_modulation_nch(hidden / 512, grid, stream, cond, w_mod, mod, num_seqs, hidden,
                                 rows);
}

hipError_t launch_adaln(const uint16_t* x, uint16_t* h, const float* shift, const float* scale,
                        int64_t mod_stride, const int32_t* cu, int num_seqs, int total_tokens,
                        int hidden, float eps, hipStream_t stream) {
    if (total_tokens == 0) return hipSuccess;
    const dim3 grid((total_tokens + 3) / 4);
    return launch_adaln_nch(hidden / 512, grid, stream, x, h, shift, scale, mod_stride, cu,
                            num_seqs, total_tokens, hidden, eps);
}

}  // namespace h3
