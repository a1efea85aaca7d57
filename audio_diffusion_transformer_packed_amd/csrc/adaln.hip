// AdaLN for the packed sequence ("MiniMax H3 FastH3 real-time serving with
// vLLM-Omni", section "System-wide optimizations in vLLM-Omni", fused DiT
// operators bullet: modulation and normalization fused).
//
//  * modulation GEMV: mod[b, :] = cond[b, :] . W_mod^T in fp32; HBM-bound on
//    the 6C x C weight, one wave per weight row (streamed once), every
//    segment's cond (staged in LDS per workgroup) applied to the row while
//    it is in registers;
//  * RMSNorm + modulate: h[t] = RMSNorm(x[t]) * (1 + scale[seg(t)]) +
//    shift[seg(t)]; one wave per row (its sum of squares is a wave
//    reduction, no workgroup barrier), two rows in flight per wave, one
//    bf16 rounding.
#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {
namespace {

constexpr int kThreads = 256;

// Segments of cond staged in LDS per pass of the modulation kernel.
constexpr int kCondChunk = 4;

template <int NCH>
__global__ __launch_bounds__(kThreads) void modulation_kernel(
    const uint16_t* __restrict__ cond, const uint16_t* __restrict__ w, float* __restrict__ mod,
    int num_seqs, int hidden, int rows) {
    // cond rows are shared by the workgroup's four waves: staged once in LDS
    // (kCondChunk segments per pass) instead of re-read from L2 per wave
    __shared__ __attribute__((aligned(16))) uint16_t cs[kCondChunk * NCH * 512];
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const bool active = row < rows;                 // every wave stays for the barriers
    float wr[NCH * 8];
    if (active) {
        const uint16_t* wp = w + static_cast<int64_t>(row) * hidden;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            Chunk16 c;
            c.u = load_stream16(wp + (i * 64 + lane) * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) wr[i * 8 + e] = bf2f(c.h[e]);
        }
    }
    for (int b0 = 0; b0 < num_seqs; b0 += kCondChunk) {
        const int nb = min(kCondChunk, num_seqs - b0);
        __syncthreads();
        for (int c = threadIdx.x; c < nb * hidden / 8; c += kThreads)
            reinterpret_cast<uint4*>(cs)[c] =
                *reinterpret_cast<const uint4*>(cond + static_cast<int64_t>(b0) * hidden + 8 * c);
        __syncthreads();
        if (!active) continue;
        for (int b = 0; b < nb; ++b) {
            const uint16_t* cp = cs + b * hidden;
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                Chunk16 c;
                c.u = *reinterpret_cast<const uint4*>(cp + (i * 64 + lane) * 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = fmaf(bf2f(c.h[e]), wr[i * 8 + e], acc);
            }
            acc = wave_sum(acc);
            if (lane == 0) mod[static_cast<int64_t>(b0 + b) * rows + row] = acc;
        }
    }
}

// RMSNorm + modulate, one wave per row: lane i owns 16-byte chunks i,
// i + 64, ... (NCH = hidden / 512 of them) of the row, so the row's sum of
// squares is a wave reduction and no workgroup barrier stands between a
// wave's loads and its stores. Each wave takes kRowsPerWave consecutive rows
// and issues all of their loads before the first reduction. The lane's
// shift / scale values stay in registers across its rows (reloaded only
// where a row changes segment) when they fit (NCH <= 8), otherwise they are
// read per row from cache. x and h are streamed with nontemporal loads /
// stores (each byte is touched once). At 57,960 x 3072 with the Infinity
// Cache flushed this runs at ~0.9x of a plain device copy of the same bytes.
constexpr int kRowsPerWave = 2;
constexpr int kAdalnWaves = 4;

// With MX the output is MXFP8 instead of bf16 (codes into h, E8M0 scales
// into hsc, K-step-major with total_tokens rows; "MiniMax H3 on Ascend 950PR
// / 950DT", MXFP8 online quantization): a 32-element block is the 4 chunks
// of 4 consecutive lanes, quantised from the fp32 values.
template <int NCH, bool MX>
__global__ __launch_bounds__(64 * kAdalnWaves) void adaln_kernel(
    const uint16_t* __restrict__ x, void* __restrict__ hout, uint8_t* __restrict__ hsc,
    const float* __restrict__ shift, const float* __restrict__ scale, int64_t mod_stride,
    const int32_t* __restrict__ cu, int num_seqs, int total_tokens, float eps) {
    constexpr int hidden = NCH * 512;
    constexpr bool kCacheMod = NCH <= 8;
    const int lane = threadIdx.x & 63;
    const int64_t t0 =
        (static_cast<int64_t>(blockIdx.x) * kAdalnWaves + (threadIdx.x >> 6)) * kRowsPerWave;
    Chunk16 xc[kRowsPerWave][NCH];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
        for (int i = 0; i < NCH; ++i)
            if (t0 + r < total_tokens)
                xc[r][i].u = load_stream16(x + (t0 + r) * hidden + (i * 64 + lane) * 8);
    int seg_loaded = -1;
    float shv[kCacheMod ? NCH : 1][8], scv[kCacheMod ? NCH : 1][8];
    auto load_mod = [&](int seg, int i, float (&sh)[8], float (&sc)[8]) __attribute__((always_inline)) {
        const float* shp = shift + static_cast<int64_t>(seg) * mod_stride + (i * 64 + lane) * 8;
        const float* scp = scale + static_cast<int64_t>(seg) * mod_stride + (i * 64 + lane) * 8;
        const float4 sh0 = *reinterpret_cast<const float4*>(shp);
        const float4 sh1 = *reinterpret_cast<const float4*>(shp + 4);
        const float4 sc0 = *reinterpret_cast<const float4*>(scp);
        const float4 sc1 = *reinterpret_cast<const float4*>(scp + 4);
        sh[0] = sh0.x; sh[1] = sh0.y; sh[2] = sh0.z; sh[3] = sh0.w;
        sh[4] = sh1.x; sh[5] = sh1.y; sh[6] = sh1.z; sh[7] = sh1.w;
        sc[0] = 1.0f + sc0.x; sc[1] = 1.0f + sc0.y; sc[2] = 1.0f + sc0.z; sc[3] = 1.0f + sc0.w;
        sc[4] = 1.0f + sc1.x; sc[5] = 1.0f + sc1.y; sc[6] = 1.0f + sc1.z; sc[7] = 1.0f + sc1.w;
    };
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
        const int64_t t = t0 + r;
        if (t >= total_tokens) break;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float f = bf2f(xc[r][i].h[e]);
                ss = fmaf(f, f, ss);
            }
        ss = wave_sum(ss);
        const float rinv = 1.0f / sqrtf(fmaf(ss, 1.0f / hidden, eps));
        const int seg = num_seqs == 1 ? 0 : find_segment(cu, num_seqs, t);
        if (kCacheMod && seg != seg_loaded) {
#pragma unroll
            for (int i = 0; i < (kCacheMod ? NCH : 1); ++i) load_mod(seg, i, shv[i], scv[i]);
            seg_loaded = seg;
        }
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            float sh[8], sc[8];
            if (kCacheMod) {
#pragma unroll
                for (int e = 0; e < 8; ++e) { sh[e] = shv[kCacheMod ? i : 0][e]; sc[e] = scv[kCacheMod ? i : 0][e]; }
            } else {
                load_mod(seg, i, sh, sc);
            }
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = fmaf(bf2f(xc[r][i].h[e]) * rinv, sc[e], sh[e]);
            if constexpr (MX) {
                float am = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(o[e]));
                am = fmaxf(am, __shfl_xor(am, 1, 64));
                am = fmaxf(am, __shfl_xor(am, 2, 64));
                const uint32_t sb = mx_scale_byte(am);
                const float inv = mx_inv_scale(sb);
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] *= inv;
                const int ch = i * 64 + lane;
                *reinterpret_cast<uint2*>(static_cast<uint8_t*>(hout) + t * hidden + ch * 8) = mx_codes8(o);
                if ((lane & 3) == 0) hsc[mx_scale_offset(t, ch >> 2, total_tokens)] = static_cast<uint8_t>(sb);
            } else {
                Chunk16 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out.w[e] = pack_bf16x2(o[2 * e], o[2 * e + 1]);
                store_stream16(static_cast<uint16_t*>(hout) + t * hidden + (i * 64 + lane) * 8, out.u);
            }
        }
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

template <bool MX, typename... Args>
hipError_t launch_adaln_nch(int nch, dim3 grid, hipStream_t stream, Args... args) {
    switch (nch) {
#define H3_ADALN_CASE(N)                                                                       \
    case N:                                                                                  \
        hipLaunchKernelGGL((adaln_kernel<N, MX>), grid, dim3(64 * kAdalnWaves), 0, stream, args...); \
        break;
        H3_ADALN_CASE(1) H3_ADALN_CASE(2) H3_ADALN_CASE(3) H3_ADALN_CASE(4)
        H3_ADALN_CASE(5) H3_ADALN_CASE(6) H3_ADALN_CASE(7) H3_ADALN_CASE(8)
        H3_ADALN_CASE(9) H3_ADALN_CASE(10) H3_ADALN_CASE(11) H3_ADALN_CASE(12)
        H3_ADALN_CASE(13) H3_ADALN_CASE(14) H3_ADALN_CASE(15) H3_ADALN_CASE(16)
#undef H3_ADALN_CASE
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
    if (hidden % 512 != 0 || hidden > 8192) return hipErrorInvalidValue;
    constexpr int rows_per_block = kRowsPerWave * kAdalnWaves;
    const dim3 grid((total_tokens + rows_per_block - 1) / rows_per_block);
    return launch_adaln_nch<false>(hidden / 512, grid, stream, x, static_cast<void*>(h),
                                   static_cast<uint8_t*>(nullptr), shift, scale, mod_stride, cu,
                                   num_seqs, total_tokens, eps);
}

hipError_t launch_adaln_mx(const uint16_t* x, uint8_t* h8, uint8_t* h_sc, const float* shift,
                           const float* scale, int64_t mod_stride, const int32_t* cu, int num_seqs,
                           int total_tokens, int hidden, float eps, hipStream_t stream) {
    if (total_tokens == 0) return hipSuccess;
    if (hidden % 512 != 0 || hidden > 8192) return hipErrorInvalidValue;
    constexpr int rows_per_block = kRowsPerWave * kAdalnWaves;
    const dim3 grid((total_tokens + rows_per_block - 1) / rows_per_block);
    return launch_adaln_nch<true>(hidden / 512, grid, stream, x, static_cast<void*>(h8), h_sc, shift,
                                  scale, mod_stride, cu, num_seqs, total_tokens, eps);
}

}  // namespace h3
