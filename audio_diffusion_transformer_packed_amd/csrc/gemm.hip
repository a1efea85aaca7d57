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
// Tiling (CDNA4): 128 x 128 x 64 workgroup tile, four waves in a 2 x 2
// arrangement, each wave 64 x 64 = 2 x 2 blocks of v_mfma_f32_32x32x16_bf16.
// A and W tiles are staged in LDS (rows padded to 72 elements), double
// buffered, with the next K-step's global loads in flight during the
// current step. For SwiGLU the W tile interleaves 32-row blocks of Wg and Wu
// so that each wave holds the gate and up accumulators of the same outputs.
#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;      // rows of the W tile
constexpr int kBK = 64;
constexpr int kStride = kBK + 8;
constexpr int kThreads = 256;
constexpr int kTileElems = (kBM + kBN) * kStride;

template <int EPI>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
    const uint16_t* __restrict__ W2, uint16_t* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    const uint16_t* __restrict__ res, const float* __restrict__ gate, int64_t gate_stride,
    const int32_t* __restrict__ cu, int num_seqs) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kTileElems];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int wm = wave & 1;
    const int wn = wave >> 1;

    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
    constexpr int OUT_N = EPI == kEpiSwiGLU ? kBN / 2 : kBN;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * OUT_N;

    // Global source row of each staged tile row handled by this thread.
    // Chunk ci = tid + 256 i covers tile row ci / 8, 16-byte column ci % 8.
    const uint16_t* a_src[4];
    const uint16_t* w_src[4];
    bool a_ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ci = tid + i * kThreads;
        const int r = ci >> 3;
        const int c = ci & 7;
        const int64_t am = m0 + r;
        a_ok[i] = am < M;
        a_src[i] = A + (a_ok[i] ? am : 0) * K + 8 * c;
        if (EPI == kEpiSwiGLU) {
            const int part = (r & 63) >> 5;         // 0: gate rows, 1: up rows
            const int64_t wrow = n0 + 32 * (r >> 6) + (r & 31);
            w_src[i] = (part ? W2 : W) + wrow * K + 8 * c;
        } else {
            w_src[i] = W + (n0 + r) * K + 8 * c;
        }
    }

    uint4 areg[4], wreg[4];
    auto load = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            areg[i] = a_ok[i] ? *reinterpret_cast<const uint4*>(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
            wreg[i] = *reinterpret_cast<const uint4*>(w_src[i] + k0);
        }
    };
    auto store = [&](int buf) {
        uint16_t* al = lds + buf * kTileElems;
        uint16_t* wl = al + kBM * kStride;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ci = tid + i * kThreads;
            const int r = ci >> 3;
            const int c = ci & 7;
            *reinterpret_cast<uint4*>(al + r * kStride + 8 * c) = areg[i];
            *reinterpret_cast<uint4*>(wl + r * kStride + 8 * c) = wreg[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    const int64_t ksteps = K / kBK;
    load(0);
    store(0);
    __syncthreads();
    for (int64_t kt = 0; kt < ksteps; ++kt) {
        const int buf = static_cast<int>(kt & 1);
        const bool has_next = kt + 1 < ksteps;
        if (has_next) load((kt + 1) * kBK);
        const uint16_t* al = lds + buf * kTileElems;
        const uint16_t* wl = al + kBM * kStride;
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            Chunk16 af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                af[i].u = *reinterpret_cast<const uint4*>(al + (64 * wm + 32 * i + l32) * kStride + 16 * ks + 8 * g);
                bf[i].u = *reinterpret_cast<const uint4*>(wl + (64 * wn + 32 * i + l32) * kStride + 16 * ks + 8 * g);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(af[i].b, bf[j].b, acc[i][j]);
        }
        if (has_next) store(buf ^ 1);
        __syncthreads();
    }

    // Epilogue. acc[i][j] register r holds row 64wm + 32i + 8(r/4) + 4g + r%4,
    // column (of the W tile) 64wn + 32j + l32.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
            if (m >= M) continue;
            if (EPI == kEpiSwiGLU) {
                const int64_t n = n0 + 32 * wn + l32;
                const float gv = acc[i][0][r];
                const float uv = acc[i][1][r];
                const float s = gv / (1.0f + __expf(-gv));
                Y[m * N + n] = f2bf(s * uv);
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int64_t n = n0 + 64 * wn + 32 * j + l32;
                    if (EPI == kEpiStore) {
                        Y[m * N + n] = f2bf(acc[i][j][r]);
                    } else {
                        const int seg = num_seqs == 1 ? 0 : find_segment(cu, num_seqs, m);
                        const float gt = gate[static_cast<int64_t>(seg) * gate_stride + n];
                        Y[m * N + n] = f2bf(fmaf(gt, acc[i][j][r], bf2f(res[m * N + n])));
                    }
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(int epilogue, const uint16_t* a, const uint16_t* w, const uint16_t* w2,
                       uint16_t* y, int64_t m, int64_t n, int64_t k, const uint16_t* res,
                       const float* gate, int64_t gate_stride, const int32_t* cu,
                       int num_seqs, hipStream_t stream) {
    if (m == 0) return hipSuccess;
    const int out_n = epilogue == kEpiSwiGLU ? kBN / 2 : kBN;
    const dim3 grid(static_cast<unsigned>(n / out_n), static_cast<unsigned>((m + kBM - 1) / kBM));
    switch (epilogue) {
        case kEpiStore:
            hipLaunchKernelGGL(gemm_kernel<kEpiStore>, grid, dim3(kThreads), 0, stream, a, w, w2,
                               y, m, n, k, res, gate, gate_stride, cu, num_seqs);
            break;
        case kEpiSwiGLU:
            hipLaunchKernelGGL(gemm_kernel<kEpiSwiGLU>, grid, dim3(kThreads), 0, stream, a, w, w2,
                               y, m, n, k, res, gate, gate_stride, cu, num_seqs);
            break;
        default:
            hipLaunchKernelGGL(gemm_kernel<kEpiGatedResidual>, grid, dim3(kThreads), 0, stream, a,
                               w, w2, y, m, n, k, res, gate, gate_stride, cu, num_seqs);
            break;
    }
    return hipGetLastError();
}

}  // namespace h3
