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
// One thread owns one 16-byte chunk (8 dims) of q and the same chunk of k,
// D/8 consecutive lanes one (token, head) vector, so every wave access is
// 1 KB of contiguous heads and each thread issues exactly two loads and two
// stores (the pattern that streams closest to the HBM copy rate), all
// nontemporal since each byte is touched once. The
// rotation rates theta^(-2j/d_axis) / (2 pi) come from a host-computed table
// in the kernel arguments; the angle in revolutions is formed and reduced to
// [-1/2, 1/2] in fp64 and fed to the hardware sin / cos (v_sin_f32 and
// v_cos_f32 take revolutions); the rotation itself is fp32 and the only
// rounding to bf16 is the final store.
#include <math.h>

#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {
namespace {

constexpr int kThreads = 256;

struct RopeRates {
    double rev[64];      // pair p of the head dim: rate in revolutions per position
    int axis[64];        // 0, 1, 2: which position (t, h, w) drives pair p
};

template <int D>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(
    uint16_t* __restrict__ q, uint16_t* __restrict__ k, int64_t qs, int64_t ks,
    const uint16_t* __restrict__ w_q, const uint16_t* __restrict__ w_k,
    const int32_t* __restrict__ grid, int64_t num_vec, int num_heads, RopeRates rr, float eps) {
    constexpr int LANES = D / 8;                 // lanes per (token, head)
    constexpr int GROUPS = kThreads / LANES;     // vectors per block
    const int tid = threadIdx.x;
    const int j = tid % LANES;                   // dims [8j, 8j + 8)
    const int64_t vec = static_cast<int64_t>(blockIdx.x) * GROUPS + tid / LANES;
    if (vec >= num_vec) return;                  // whole groups leave together
    const int64_t t = vec / num_heads;
    const int h = static_cast<int>(vec - t * num_heads);
    uint16_t* qp = q + t * qs + static_cast<int64_t>(h) * D + 8 * j;
    uint16_t* kp = k + t * ks + static_cast<int64_t>(h) * D + 8 * j;
    Chunk16 qc, kc, wq, wk;
    qc.u = load_stream16(qp);
    kc.u = load_stream16(kp);
    wq.u = *reinterpret_cast<const uint4*>(w_q + 8 * j);
    wk.u = *reinterpret_cast<const uint4*>(w_k + 8 * j);
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
    const float rq = 1.0f / sqrtf(fmaf(sq, 1.0f / D, eps));
    const float rk = 1.0f / sqrtf(fmaf(sk, 1.0f / D, eps));

#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int pp = 4 * j + p;
        const int ax = rr.axis[pp];
        const int pa = ax == 0 ? pos3[0] : (ax == 1 ? pos3[1] : pos3[2]);
        double rev = static_cast<double>(pa) * rr.rev[pp];
        rev -= rint(rev);
        const float rf = static_cast<float>(rev);
        const float sn = __builtin_amdgcn_sinf(rf);
        const float cs = __builtin_amdgcn_cosf(rf);
        const float qu = xq[2 * p] * rq * bf2f(wq.h[2 * p]);
        const float qv = xq[2 * p + 1] * rq * bf2f(wq.h[2 * p + 1]);
        const float ku = xk[2 * p] * rk * bf2f(wk.h[2 * p]);
        const float kv = xk[2 * p + 1] * rk * bf2f(wk.h[2 * p + 1]);
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
    store_stream16(qp, oq.u);
    store_stream16(kp, ok.u);
}

}  // namespace

hipError_t launch_qk_norm_rope(uint16_t* q, uint16_t* k, int64_t qs, int64_t ks,
                               const uint16_t* w_q, const uint16_t* w_k, const int32_t* grid,
                               int total_tokens, int num_heads, int head_dim,
                               const int32_t split[3], float theta, float eps,
                               hipStream_t stream) {
    const int64_t num_vec = static_cast<int64_t>(total_tokens) * num_heads;
    if (num_vec == 0) return hipSuccess;
    // pair p covers dims (2p, 2p + 1); inside axis a's slice it is pair jj of d_a
    RopeRates rr;
    const double two_pi = 6.283185307179586476925286766559;
    for (int p = 0; p < head_dim / 2; ++p) {
        const int d = 2 * p;
        int a, jj, da;
        if (d < split[0]) { a = 0; jj = d / 2; da = split[0]; }
        else if (d < split[0] + split[1]) { a = 1; jj = (d - split[0]) / 2; da = split[1]; }
        else { a = 2; jj = (d - split[0] - split[1]) / 2; da = split[2]; }
        rr.axis[p] = a;
        rr.rev[p] = pow(static_cast<double>(theta), -2.0 * jj / da) / two_pi;
    }
    const int groups = kThreads / (head_dim / 8);
    const int64_t blocks = (num_vec + groups - 1) / groups;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    if (head_dim == 128) {
        hipLaunchKernelGGL(qk_norm_rope_kernel<128>, dim3(static_cast<unsigned>(blocks)),
                           dim3(kThreads), 0, stream, q, k, qs, ks, w_q, w_k, grid, num_vec,
                           num_heads, rr, eps);
    } else {
        hipLaunchKernelGGL(qk_norm_rope_kernel<64>, dim3(static_cast<unsigned>(blocks)),
                           dim3(kThreads), 0, stream, q, k, qs, ks, w_q, w_k, grid, num_vec,
                           num_heads, rr, eps);
    }
    return hipGetLastError();
}

}  // namespace h3
