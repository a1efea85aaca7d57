// Varlen bookkeeping on the device: segment id per token, query-tile offsets
// per segment and the attention work list. Padding never enters the list:
// only the valid tokens of each packed segment are scheduled (packed-sequence
// attention over valid tokens, "MiniMax H3 FastH3 real-time serving with
// vLLM-Omni", section "System-wide optimizations in vLLM-Omni").
//
// Work-list order: segments by descending length (ties by index), then head,
// then query tile. Consecutive items therefore share one (segment, head) and
// stream the same K/V, which keeps concurrently resident workgroups on the
// same keys, and the longest segments start first.
#include "h3_common.hpp"
#include "h3_internal.hpp"

namespace h3 {
namespace {

constexpr int kThreads = 1024;

__device__ int block_exclusive_scan(int v, int* sm, int* total) {
    const int t = threadIdx.x;
    sm[t] = v;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        int add = t >= off ? sm[t - off] : 0;
        __syncthreads();
        sm[t] += add;
        __syncthreads();
    }
    int incl = sm[t];
    *total = sm[kThreads - 1];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(kThreads) void schedule_kernel(
    const int32_t* __restrict__ cu, int num_seqs, int num_heads, int block_m,
    int32_t* __restrict__ tile_cu, int32_t* __restrict__ items, int64_t capacity,
    int32_t* __restrict__ order, int32_t* __restrict__ rank_prefix) {
    __shared__ int sm[kThreads];
    __shared__ int total_sm;
    const int t = threadIdx.x;

    // 1. rank of each segment in (length desc, index asc) order
    for (int s = t; s < num_seqs; s += kThreads) {
        const int len = cu[s + 1] - cu[s];
        int rank = 0;
        for (int s2 = 0; s2 < num_seqs; ++s2) {
            const int len2 = cu[s2 + 1] - cu[s2];
            rank += (len2 > len) || (len2 == len && s2 < s);
        }
        order[rank] = s;
    }
    __syncthreads();

    // 2. exclusive prefix of tile counts, by rank and by segment index
    int carry_rank = 0, carry_seg = 0;
    for (int base = 0; base < num_seqs; base += kThreads) {
        const int i = base + t;
        int tiles_rank = 0, tiles_seg = 0;
        if (i < num_seqs) {
            const int sr = order[i];
            tiles_rank = (cu[sr + 1] - cu[sr] + block_m - 1) / block_m;
            tiles_seg = (cu[i + 1] - cu[i] + block_m - 1) / block_m;
        }
        int tot;
        int ex = block_exclusive_scan(tiles_rank, sm, &tot);
        if (i < num_seqs) rank_prefix[i] = carry_rank + ex;
        carry_rank += tot;
        __syncthreads();
        ex = block_exclusive_scan(tiles_seg, sm, &tot);
        if (i < num_seqs && tile_cu) tile_cu[i] = carry_seg + ex;
        carry_seg += tot;
        __syncthreads();
    }
    if (t == 0) {
        rank_prefix[num_seqs] = carry_rank;
        if (tile_cu) tile_cu[num_seqs] = carry_seg;
        total_sm = carry_rank;
    }
    __syncthreads();

    // 3. items, one per (rank, head, tile), written in list order
    const int64_t count = static_cast<int64_t>(total_sm) * num_heads;
    const int64_t limit = count < capacity ? count : capacity;
    for (int64_t idx = t; idx < limit; idx += kThreads) {
        // largest rank r with num_heads * rank_prefix[r] <= idx
        int lo = 0, hi = num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (static_cast<int64_t>(rank_prefix[mid]) * num_heads <= idx) lo = mid; else hi = mid - 1;
        }
        const int s = order[lo];
        const int tiles = rank_prefix[lo + 1] - rank_prefix[lo];
        const int64_t within = idx - static_cast<int64_t>(rank_prefix[lo]) * num_heads;
        const int h = static_cast<int>(within / tiles);
        const int tile = static_cast<int>(within % tiles);
        const int len = cu[s + 1] - cu[s];
        const int off = tile * block_m;
        int4 it;
        it.x = h;
        it.y = s;
        it.z = cu[s] + off;
        it.w = min(block_m, len - off);
        reinterpret_cast<int4*>(items)[idx] = it;
    }
}

__global__ void seg_id_kernel(const int32_t* __restrict__ cu, int num_seqs, int total_tokens,
                              int32_t* __restrict__ seg_id) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t < total_tokens) seg_id[t] = find_segment(cu, num_seqs, t);
}

}  // namespace

size_t bookkeeping_scratch_bytes(int num_seqs) {
    // order[num_seqs] + rank_prefix[num_seqs + 1], rounded to 256 bytes
    size_t b = sizeof(int32_t) * (2 * static_cast<size_t>(num_seqs) + 1);
    return (b + 255) & ~static_cast<size_t>(255);
}

const int32_t* bookkeeping_rank_prefix(const void* scratch, int num_seqs) {
    return static_cast<const int32_t*>(scratch) + num_seqs;
}

hipError_t launch_bookkeeping(const int32_t* cu, int num_seqs, int total_tokens, int num_heads,
                              int block_m, int32_t* seg_id, int32_t* tile_cu, int32_t* items,
                              int64_t items_capacity, void* scratch, hipStream_t stream) {
    if (num_seqs <= 0) return hipSuccess;
    int32_t* order = static_cast<int32_t*>(scratch);
    int32_t* rank_prefix = order + num_seqs;
    if (items != nullptr || tile_cu != nullptr) {
        hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kThreads), 0, stream, cu, num_seqs,
                           num_heads, block_m, tile_cu, items, items ? items_capacity : 0,
                           order, rank_prefix);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (seg_id != nullptr && total_tokens > 0) {
        const int threads = 256;
        const int blocks = (total_tokens + threads - 1) / threads;
        hipLaunchKernelGGL(seg_id_kernel, dim3(blocks), dim3(threads), 0, stream, cu, num_seqs,
                           total_tokens, seg_id);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace h3
