// Key-block selection of the block-sparse attention path ("MiniMax H3 on
// Ascend 950PR / 950DT", section "Recommended lossy configuration (Ascend
// 950PR / 950DT)": EQBSA block-sparse attention with Q/K in INT8 and V in
// FP8 at sparsity 0.8; the page names the method and its sparsity only).
//
// Reading: query blocks are the 256-row attention work items, key blocks
// the 64-key tiles, both aligned to the segment start. A query block keeps
// keep(n) = max(1, n - floor(n p / 1000)) of its segment's n key blocks
// (p = sparsity in thousandths): those with the highest logit between the
// block means of the INT8 codes,
//   score_j = ((sum over the query block's 64-row blocks b, ascending, of
//               sq_b * I_bj) * sk_j) / n_j,
// I_bj the exact integer dot product of the code sums of Q block b and key
// block j, sq / sk the stored fp32 scales, n_j the keys in block j; each
// operation one float64 rounding in this order (no contraction), equal
// scores going to the lower block index. The kept indices are written in
// ascending order, the order the attention kernel visits them.
//
// One workgroup of 256 threads per work item: the query block's code sums
// (up to 4 x 128, int16) go to LDS; each thread scores four key blocks at a
// time, j = tid + 256 m, reading each key block's 128 code sums (256 B, from L2,
// every query block of the head reads the same sums); the (score, j)
// pairs are sorted in LDS by a bitonic network, the first keep(n) marked,
// and the marks compacted in ascending j by a workgroup scan.
#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {
namespace {

constexpr int kD = 128;
constexpr int kBN = 64;
constexpr int kThreads = 256;

typedef short s16x2 __attribute__((ext_vector_type(2)));

// acc + a.lo b.lo + a.hi b.hi for two packed int16 pairs, exact (no clamp)
__device__ __forceinline__ int dot2(uint32_t a, uint32_t b, int acc) {
    return __builtin_amdgcn_sdot2(__builtin_bit_cast(s16x2, a), __builtin_bit_cast(s16x2, b), acc, false);
}

__device__ __forceinline__ bool before(double ka, int ia, double kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

__global__ __launch_bounds__(kThreads) void bsa_select_kernel(
    const int16_t* __restrict__ qsum, const int16_t* __restrict__ ksum, const float* __restrict__ qsc,
    const float* __restrict__ ksc, const int32_t* __restrict__ cu, const int32_t* __restrict__ tb,
    const int4* __restrict__ items, int num_seqs, int total_tokens, int num_heads, int64_t num_tiles,
    int sp_permille, int64_t list_stride, int32_t* __restrict__ lists, int npow_max) {
#pragma clang fp contract(off)
    __shared__ __attribute__((aligned(16))) int16_t pq[4][kD];
    // sort arrays sized at launch for the longest segment (npow_max slots:
    // 8 + 2 + 1 bytes each), so short segments leave room for more
    // workgroups per CU
    extern __shared__ __attribute__((aligned(16))) char dyn[];
    double* key = reinterpret_cast<double*>(dyn);
    uint16_t* idx = reinterpret_cast<uint16_t*>(dyn + 8 * npow_max);
    uint8_t* mark = reinterpret_cast<uint8_t*>(dyn + 10 * npow_max);
    __shared__ int32_t part[kThreads];

    const int tid = threadIdx.x;
    const int4 it = items[blockIdx.x];
    const int head = it.x, seg = it.y, q0 = it.z, qlen = it.w;
    if (seg < 0 || seg >= num_seqs || head < 0 || head >= num_heads) return;
    const int kv0 = max(0, cu[seg]), kv1 = min(total_tokens, cu[seg + 1]);
    if (qlen <= 0 || q0 < kv0 || q0 + qlen > kv1 || (q0 - kv0) % (4 * kBN) != 0) return;
    const int len = kv1 - kv0;
    const int n = (len + kBN - 1) / kBN;
    if (n > npow_max) return;                         // never: npow_max covers every segment
    const int keep = max(1, n - static_cast<int>((static_cast<int64_t>(n) * sp_permille) / 1000));
    const int tbs = tb[seg];
    const int t0 = tbs + (q0 - kv0) / kBN;            // first 64-row block of the query block
    const int nb = (qlen + kBN - 1) / kBN;

    for (int i = tid; i < 4 * kD; i += kThreads)
        pq[i / kD][i % kD] = i / kD < nb ? qsum[(static_cast<int64_t>(t0 + i / kD) * num_heads + head) * kD + i % kD]
                                         : int16_t{0};
    double sq[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
        sq[b] = b < nb ? static_cast<double>(qsc[static_cast<int64_t>(t0 + b) * num_heads + head]) : 0.0;
    int npow = 1;
    while (npow < n) npow <<= 1;
    for (int j = tid; j < npow; j += kThreads) mark[j] = 0;
    __syncthreads();

    // Four key blocks per thread and pass (j = j0 + 256 m), so each LDS read
    // of the Q sums serves four blocks. |code sum| <= 64 * 127 = 8128 fits
    // int16: v_dot2_i32_i16 takes two exact products per instruction, 16
    // products fit an int32 partial (< 1.06e9) and the partials add exactly
    // in float64 (every value an integer below 2^53).
    // K sums are channel chunk-major ([H][16][T][8]): chunk c of key block j
    // is 16 bytes at ((head * 16 + c) * T + tbs + j) * 8, so the lanes of a
    // wave (consecutive j) read 1 KB contiguous per load instruction
    const uint4* kbase = reinterpret_cast<const uint4*>(ksum) + static_cast<int64_t>(head) * (kD / 8) * num_tiles + tbs;
    for (int j0 = tid; j0 < npow; j0 += 4 * kThreads) {
        const uint4* kp[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) kp[m] = kbase + min(j0 + kThreads * m, n - 1);
        double dot[4][4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int b = 0; b < 4; ++b) dot[m][b] = 0.0;
        for (int c0 = 0; c0 < kD; c0 += 16) {
            int part[4][4];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int b = 0; b < 4; ++b) part[m][b] = 0;
#pragma unroll
            for (int c = c0; c < c0 + 16; c += 8) {
                uint4 pb[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) pb[b] = *reinterpret_cast<const uint4*>(&pq[b][c]);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const uint4 kv = kp[m][static_cast<int64_t>(c / 8) * num_tiles];
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        part[m][b] = dot2(pb[b].x, kv.x, part[m][b]);
                        part[m][b] = dot2(pb[b].y, kv.y, part[m][b]);
                        part[m][b] = dot2(pb[b].z, kv.z, part[m][b]);
                        part[m][b] = dot2(pb[b].w, kv.w, part[m][b]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int b = 0; b < 4; ++b) dot[m][b] += static_cast<double>(part[m][b]);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int j = j0 + kThreads * m;
            if (j >= npow) continue;
            double score = -INFINITY;
            if (j < n) {
                double acc = 0.0;
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    if (b < nb) acc = acc + sq[b] * dot[m][b];
                const int nj = min(kBN, len - kBN * j);
                score = (acc * static_cast<double>(ksc[static_cast<int64_t>(tbs + j) * num_heads + head])) /
                        static_cast<double>(nj);
            }
            key[j] = score;
            idx[j] = static_cast<uint16_t>(j);      // pads (j >= n) sort after every real block
        }
    }
    __syncthreads();

    // bitonic sort of npow (score, index) pairs into "before" order; strides
    // are powers of two, so the pair index is shifts and masks
    for (int size = 2; size <= npow; size <<= 1) {
        for (int ls = __builtin_ctz(static_cast<unsigned>(size)) - 1; ls >= 0; --ls) {
            const int stride = 1 << ls;
            for (int i = tid; i < npow / 2; i += kThreads) {
                const int lo = ((i >> ls) << (ls + 1)) | (i & (stride - 1));
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const double klo = key[lo], khi = key[hi];
                const int ilo = idx[lo], ihi = idx[hi];
                if (before(khi, ihi, klo, ilo) == up) {
                    key[lo] = khi;
                    key[hi] = klo;
                    idx[lo] = static_cast<uint16_t>(ihi);
                    idx[hi] = static_cast<uint16_t>(ilo);
                }
            }
            __syncthreads();
        }
    }
    for (int r = tid; r < keep; r += kThreads) mark[idx[r]] = 1;
    __syncthreads();

    // ascending compaction: thread tid owns blocks [tid * per, (tid + 1) * per)
    const int per = (n + kThreads - 1) / kThreads;
    const int j0 = min(n, tid * per), j1 = min(n, j0 + per);
    int cnt = 0;
    for (int j = j0; j < j1; ++j) cnt += mark[j];
    part[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        const int add = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    int pos = part[tid] - cnt;
    int32_t* out = lists + (static_cast<int64_t>(head) * num_tiles + t0) * list_stride;
    for (int j = j0; j < j1; ++j)
        if (mark[j]) out[pos++] = j;
}

}  // namespace

hipError_t launch_bsa_select(const int16_t* qsum, const int16_t* ksum, const float* qsc, const float* ksc,
                             const int32_t* cu, const int32_t* tb, const int32_t* items, int64_t num_items,
                             int num_seqs, int total_tokens, int num_heads, int64_t num_tiles,
                             int sp_permille, int64_t list_stride, int32_t* lists, int max_key_blocks,
                             hipStream_t stream) {
    if (num_items <= 0) return hipSuccess;
    if (max_key_blocks > kBsaMaxKeyBlocks) return hipErrorInvalidValue;
    int npow_max = 1;
    while (npow_max < max_key_blocks) npow_max <<= 1;
    hipLaunchKernelGGL(bsa_select_kernel, dim3(static_cast<unsigned>(num_items)), dim3(kThreads),
                       static_cast<unsigned>(11 * npow_max), stream,
                       qsum, ksum, qsc, ksc, cu, tb, reinterpret_cast<const int4*>(items), num_seqs,
                       total_tokens, num_heads, num_tiles, sp_permille, list_stride, lists, npow_max);
    return hipGetLastError();
}

}  // namespace h3
