// AdaLN for the packed sequence ("MiniMax H3 FastH3 real-time serving with
// vLLM-Omni", section "System-wide optimizations in vLLM-Omni", fused DiT
// operators bullet: modulation and normalization fused).
//
//  * modulation GEMV: mod[b, :] = cond[b, :] . W_mod^T in fp32; HBM-bound on
//    the 6C x C weight, one wave per weight row (streamed once), every
//    segment's cond applied to the row while it is in registers;
//  * RMSNorm + modulate: h[t] = RMSNorm(x[t]) * (1 + scale[seg(t)]) +
//    shift[seg(t)]; one wave per row (its sum of squares is a wave
//    reduction), the modulation values of the workgroup's segment staged in
//    LDS, one bf16 rounding.
#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {
namespace {

constexpr int kThreads = 256;

// Modulation GEMV, one wave per weight row: the row (hidden bf16) is loaded
// once into registers, then every segment's cond row is read (a 6 KB row at
// hidden 3072, served from L2 after the first wave) and dotted with it. No
// LDS and no barriers: at 6 x 3072 x 3072 this measured 20 us (70 % of
// 8 TB/s) against 24 us with cond staged in LDS behind workgroup barriers.
template <int NCH>
__global__ __launch_bounds__(kThreads) void modulation_kernel(
    const uint16_t* __restrict__ cond, const uint16_t* __restrict__ w, float* __restrict__ mod,
    int num_seqs, int hidden, int rows) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (row >= rows) return;                        // whole wave: no barrier below
    Chunk16 wr[NCH];
    const uint16_t* wp = w + static_cast<int64_t>(row) * hidden;
#pragma unroll
    for (int i = 0; i < NCH; ++i) wr[i].u = load_stream16(wp + (i * 64 + lane) * 8);
    for (int b = 0; b < num_seqs; ++b) {
        const uint16_t* cp = cond + static_cast<int64_t>(b) * hidden;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            Chunk16 c;
            c.u = *reinterpret_cast<const uint4*>(cp + (i * 64 + lane) * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf(bf2f(c.h[e]), bf2f(wr[i].h[e]), acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) mod[static_cast<int64_t>(b) * rows + row] = acc;
    }
}

// RMSNorm + modulate, one wave per row: lane i owns 16-byte chunks i,
// i + 64, ... (NCH = hidden / 512 of them) of the row, so the row's sum of
// squares is a wave reduction. A workgroup of kAdalnWaves waves takes
// kAdalnWaves consecutive rows; it stages (1 + scale) and shift of its first
// row's segment in LDS (one read of 2 x hidden floats shared by all its
// waves), and a row of another segment (only where a workgroup straddles a
// segment boundary) reads its own from memory instead, in the same fp32
// arithmetic. One row per wave keeps the register count low, so many waves
// are resident and many loads are in flight. x and h are streamed with
// nontemporal loads / stores (each byte is touched once). At 57,960 x 3072
// with the Infinity Cache flushed: 121 us (73 % of 8 TB/s) against 126 us
// for two rows per wave with the modulation values held in registers.
constexpr int kAdalnWaves = 8;

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
    __shared__ float4 lsh[hidden / 4], lsc[hidden / 4];
    const int lane = threadIdx.x & 63;
    const int64_t tb = static_cast<int64_t>(blockIdx.x) * kAdalnWaves;   // first row of the workgroup
    const int64_t t = tb + (threadIdx.x >> 6);
    Chunk16 xc[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i)
        if (t < total_tokens) xc[i].u = load_stream16(x + t * hidden + (i * 64 + lane) * 8);
    const int bseg = num_seqs == 1 ? 0 : find_segment(cu, num_seqs, tb);
    for (int c = threadIdx.x; c < hidden / 4; c += 64 * kAdalnWaves) {
        const float4 a = reinterpret_cast<const float4*>(shift + static_cast<int64_t>(bseg) * mod_stride)[c];
        float4 b = reinterpret_cast<const float4*>(scale + static_cast<int64_t>(bseg) * mod_stride)[c];
        b.x += 1.0f; b.y += 1.0f; b.z += 1.0f; b.w += 1.0f;
        lsh[c] = a;
        lsc[c] = b;
    }
    __syncthreads();
    if (t >= total_tokens) return;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float f = bf2f(xc[i].h[e]);
            ss = fmaf(f, f, ss);
        }
    ss = wave_sum(ss);
    const float rinv = 1.0f / sqrtf(fmaf(ss, 1.0f / hidden, eps));
    const int seg = num_seqs == 1 ? 0 : find_segment(cu, num_seqs, t);
    const float4* gsh = reinterpret_cast<const float4*>(shift + static_cast<int64_t>(seg) * mod_stride);
    const float4* gsc = reinterpret_cast<const float4*>(scale + static_cast<int64_t>(seg) * mod_stride);
    const bool own = seg == bseg;                    // wave-uniform
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c4 = (i * 64 + lane) * 2;
        float4 sh0, sh1, sc0, sc1;
        if (own) {
            sh0 = lsh[c4]; sh1 = lsh[c4 + 1]; sc0 = lsc[c4]; sc1 = lsc[c4 + 1];
        } else {
            sh0 = gsh[c4]; sh1 = gsh[c4 + 1]; sc0 = gsc[c4]; sc1 = gsc[c4 + 1];
            sc0.x += 1.0f; sc0.y += 1.0f; sc0.z += 1.0f; sc0.w += 1.0f;
            sc1.x += 1.0f; sc1.y += 1.0f; sc1.z += 1.0f; sc1.w += 1.0f;
        }
        const float sh[8] = {sh0.x, sh0.y, sh0.z, sh0.w, sh1.x, sh1.y, sh1.z, sh1.w};
        const float sc[8] = {sc0.x, sc0.y, sc0.z, sc0.w, sc1.x, sc1.y, sc1.z, sc1.w};
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(bf2f(xc[i].h[e]) * rinv, sc[e], sh[e]);
        if constexpr (MX) {
            float am = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(o[e]));
            // the block's 4 lanes form a DPP quad: swap within pairs, then
            // halves (quad_perm [1,0,3,2] and [2,3,0,1]; no LDS permute)
            am = fmaxf(am, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                               __builtin_bit_cast(int, am), 0xB1, 0xF, 0xF, true)));
            am = fmaxf(am, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                               __builtin_bit_cast(int, am), 0x4E, 0xF, 0xF, true)));
            const uint32_t sb = mx_scale_byte(am);
            const float inv = mx_inv_scale(sb);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] *= inv;
            const int ch = i * 64 + lane;
            *reinterpret_cast<uint2*>(static_cast<uint8_t*>(hout) + t * hidden + ch * 8) = mx_codes8(o);
            // the four blocks of a 128-element K step are the quads of a
            // 16-lane row: each quad's byte moved to its place in the step's
            // scale dword, the row OR-combined with two DPP rotations (by 4
            // and 8 lanes), one dword store per row of lanes
            uint32_t sw = sb << (8 * ((lane >> 2) & 3));
            sw |= static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(sw), 0x124, 0xF, 0xF, false));
            sw |= static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(sw), 0x128, 0xF, 0xF, false));
            if ((lane & 15) == 0)
                *reinterpret_cast<uint32_t*>(hsc + mx_scale_offset(t, ch >> 2, total_tokens)) = sw;
        } else {
            Chunk16 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) out.w[e] = pack_bf16x2(o[2 * e], o[2 * e + 1]);
            store_stream16(static_cast<uint16_t*>(hout) + t * hidden + (i * 64 + lane) * 8, out.u);
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
    const dim3 grid((total_tokens + kAdalnWaves - 1) / kAdalnWaves);
    return launch_adaln_nch<false>(hidden / 512, grid, stream, x, static_cast<void*>(h),
                                   static_cast<uint8_t*>(nullptr), shift, scale, mod_stride, cu,
                                   num_seqs, total_tokens, eps);
}

hipError_t launch_adaln_mx(const uint16_t* x, uint8_t* h8, uint8_t* h_sc, const float* shift,
                           const float* scale, int64_t mod_stride, const int32_t* cu, int num_seqs,
                           int total_tokens, int hidden, float eps, hipStream_t stream) {
    if (total_tokens == 0) return hipSuccess;
    if (hidden % 512 != 0 || hidden > 8192) return hipErrorInvalidValue;
    const dim3 grid((total_tokens + kAdalnWaves - 1) / kAdalnWaves);
    return launch_adaln_nch<true>(hidden / 512, grid, stream, x, static_cast<void*>(h8), h_sc, shift,
                                  scale, mod_stride, cu, num_seqs, total_tokens, eps);
}

}  // namespace h3
