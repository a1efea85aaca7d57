// Fused per-head Q/K RMSNorm + 3D RoPE, in place ("FastH3 在八卡 B300 上实现
// 完整 MP4 生成快于播放时长", section "融合 DiT 算子": the Q/K normalisation
// is merged with RoPE into one kernel).
//
// For token t and head h, x = q[t, h, :] (and the same for k):
//   x <- RoPE_pos(t)(x / sqrt(mean(x^2) + eps) * w)
// RoPE rotates interleaved pairs (2j, 2j+1) of each axis slice (t, h, w) by
// pos_axis * theta^(-2j / d_axis).
//
// HBM-bound: each (token, head) is read once and written once for q and k.
// A group of D/8 lanes owns one (token, head) vector, 16 bytes per lane,
// so a wave reads and writes 1 KB (D = 128) of contiguous heads per access.
// q and k of the same (token, head) share one group, so the rotation angles
// are computed once for both. Angles are formed and range-reduced in fp64,
// the rotation itself is fp32; the only rounding to bf16 is the final store.
#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {
namespace {

constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(
    uint16_t* __restrict__ q, uint16_t* __restrict__ k, int64_t qs, int64_t ks,
    const uint16_t* __restrict__ w_q, const uint16_t* __restrict__ w_k,
    const int32_t* __restrict__ grid, int64_t num_vec, int num_heads, int s0, int s1, int s2,
    double theta, float eps) {
    constexpr int LANES = D / 8;                 // lanes per (token, head)
    constexpr int GROUPS = kThreads / LANES;     // vectors per block per step
    const int tid = threadIdx.x;
    const int j = tid % LANES;                   // dims [8j, 8j + 8)
    const int grp = tid / LANES;

    // per-lane constants: gains and, for each of the 4 pairs, axis and rate
    float gq[8], gk[8];
    {
        Chunk16 a, b;
        a.u = *reinterpret_cast<const uint4*>(w_q + 8 * j);
        b.u = *reinterpret_cast<const uint4*>(w_k + 8 * j);
#pragma unroll
        for (int e = 0; e < 8; ++e) { gq[e] = bf2f(a.h[e]); gk[e] = bf2f(b.h[e]); }
    }
    int axis[4];
    double rate[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int d = 8 * j + 2 * p;
        int a, jj, da;
        if (d < s0) { a = 0; jj = d / 2; da = s0; }
        else if (d < s0 + s1) { a = 1; jj = (d - s0) / 2; da = s1; }
        else { a = 2; jj = (d - s0 - s1) / 2; da = s2; }
        axis[p] = a;
        rate[p] = pow(theta, -2.0 * jj / da);
    }
    const double two_pi = 6.283185307179586476925286766559;
    const float inv_d = 1.0f / D;

    for (int64_t vec = static_cast<int64_t>(blockIdx.x) * GROUPS + grp; vec < num_vec;
         vec += static_cast<int64_t>(gridDim.x) * GROUPS) {
        const int64_t t = vec / num_heads;
        const int h = static_cast<int>(vec - t * num_heads);
        uint16_t* qp = q + t * qs + static_cast<int64_t>(h) * D + 8 * j;
        uint16_t* kp = k + t * ks + static_cast<int64_t>(h) * D + 8 * j;
        Chunk16 qc, kc;
        qc.u = *reinterpret_cast<const uint4*>(qp);
        kc.u = *reinterpret_cast<const uint4*>(kp);
        const int pos3[3] = {grid[3 * t + 0], grid[3 * t + 1], grid[3 * t + 2]};

        float xq[8], xk[8];
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            xq[e] = bf2f(qc.h[e]);
            xk[e] = bf2f(kc.h[e]);
            sq = fmaf(xq[e], xq[e], sq);
            sk = fmaf(xk[e], xk[e], sk);
        }
        sq = group_sum<LANES>(sq);
        sk = group_sum<LANES>(sk);
        const float rq = 1.0f / sqrtf(fmaf(sq, inv_d, eps));
        const float rk = 1.0f / sqrtf(fmaf(sk, inv_d, eps));

#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int pa = axis[p] == 0 ? pos3[0] : (axis[p] == 1 ? pos3[1] : pos3[2]);
            double ang = static_cast<double>(pa) * rate[p];
            ang -= two_pi * rint(ang / two_pi);
            float sn, cs;
            sincosf(static_cast<float>(ang), &sn, &cs);
            const float qu = xq[2 * p] * rq * gq[2 * p];
            const float qv = xq[2 * p + 1] * rq * gq[2 * p + 1];
            const float ku = xk[2 * p] * rk * gk[2 * p];
            const float kv = xk[2 * p + 1] * rk * gk[2 * p + 1];
            xq[2 * p] = qu * cs - qv * sn;
            xq[2 * p + 1] = qu * sn + qv * cs;
            xk[2 * p] = ku * cs - kv * sn;
            xk[2 * p + 1] = ku * sn + kv * cs;
        }
        Chunk16 oq, ok;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            oq.w[e] = pack_bf16x2(xq[2 * e], xq[2 * e + 1]);
            ok.w[e] = pack_bf16x2(xk[2 * e], xk[2 * e + 1]);
        }
        *reinterpret_cast<uint4*>(qp) = oq.u;
        *reinterpret_cast<uint4*>(kp) = ok.u;
    }
}

}  // namespace

hipError_t launch_qk_norm_rope(uint16_t* q, uint16_t* k, int64_t qs, int64_t ks,
                               const uint16_t* w_q, const uint16_t* w_k, const int32_t* grid,
                               int total_tokens, int num_heads, int head_dim,
                               const int32_t split[3], float theta, float eps,
                               hipStream_t stream) {
    const int64_t num_vec = static_cast<int64_t>(total_tokens) * num_heads;
    if (num_vec == 0) return hipSuccess;
    const int groups = kThreads / (head_dim / 8);
    int64_t blocks = (num_vec + groups - 1) / groups;
    const int64_t cap = 256 * 32;     // 256 CUs x 32 blocks, grid-stride beyond
    if (blocks > cap) blocks = cap;
    if (head_dim == 128) {
        hipLaunchKernelGGL(qk_norm_rope_kernel<128>, dim3(static_cast<unsigned>(blocks)),
                           dim3(kThreads), 0, stream, q, k, qs, ks, w_q, w_k, grid, num_vec,
                           num_heads, split[0], split[1], split[2], static_cast<double>(theta),
                           eps);
    } else {
        hipLaunchKernelGGL(qk_norm_rope_kernel<64>, dim3(static_cast<unsigned>(blocks)),
                           dim3(kThreads), 0, stream, q, k, qs, ks, w_q, w_k, grid, num_vec,
                           num_heads, split[0], split[1], split[2], static_cast<double>(theta),
                           eps);
    }
    return hipGetLastError();
}

}  // namespace h3
