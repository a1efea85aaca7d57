// C ABI of the packed joint audio-video DiT hot path (declared in h3dit.h).
//
// Every entry point validates all of its arguments on the host before the
// first launch (a non-OK status other than H3_ERR_HIP means nothing was
// enqueued), carves the caller's workspace, and enqueues kernels on the
// caller's stream without synchronising. The library's only state is the
// thread-local error message.
#include <math.h>

#include <cmath>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/h3dit.h"
#include "h3_internal.hpp"

// Fixed device scratch of h3_attn_varlen_noalloc (see noalloc_scratch below).
static __device__ __attribute__((aligned(256))) char scratch[H3_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

h3_status fail(h3_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

h3_status ok() { return H3_OK; }

h3_status hip_fail(hipError_t e, const char* what) {
    return fail(H3_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t b) { return (b + kAlign - 1) & ~(kAlign - 1); }

// Checks cu[0] = 0, non-decreasing, cu[B] = N.
h3_status check_cu(const int32_t* cu, int32_t num_seqs, int32_t total_tokens) {
    if (num_seqs < 0 || num_seqs > H3_MAX_SEGMENTS)
        return fail(H3_ERR_INVALID_ARGUMENT, "num_seqs=%d outside [0, %d]", num_seqs, H3_MAX_SEGMENTS);
    if (total_tokens < 0) return fail(H3_ERR_INVALID_ARGUMENT, "total_tokens=%d < 0", total_tokens);
    if (cu == nullptr) return fail(H3_ERR_INVALID_ARGUMENT, "cu_seqlens_host is NULL");
    if (cu[0] != 0) return fail(H3_ERR_INVALID_ARGUMENT, "cu_seqlens[0]=%d, expected 0", cu[0]);
    for (int32_t s = 0; s < num_seqs; ++s) {
        if (cu[s + 1] < cu[s])
            return fail(H3_ERR_INVALID_ARGUMENT, "cu_seqlens decreases at %d (%d -> %d)", s, cu[s],
                        cu[s + 1]);
    }
    if (cu[num_seqs] != total_tokens)
        return fail(H3_ERR_INVALID_ARGUMENT, "cu_seqlens[%d]=%d != total_tokens=%d", num_seqs,
                    cu[num_seqs], total_tokens);
    return ok();
}

int64_t count_items(const int32_t* cu, int32_t num_seqs, int32_t num_heads, int32_t block_m) {
    int64_t tiles = 0;
    for (int32_t s = 0; s < num_seqs; ++s) tiles += (cu[s + 1] - cu[s] + block_m - 1) / block_m;
    return tiles * num_heads;
}

// Upper bound of the item count for any cu_seqlens with these sizes.
int64_t max_items(int32_t num_seqs, int32_t total_tokens, int32_t num_heads, int32_t block_m) {
    const int64_t tiles = (static_cast<int64_t>(total_tokens) + static_cast<int64_t>(num_seqs) * (block_m - 1)) / block_m;
    return tiles * num_heads;
}

bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }

h3_status check_split(const int32_t* split, int32_t head_dim) {
    if (split == nullptr) return fail(H3_ERR_INVALID_ARGUMENT, "rope_split is NULL");
    for (int a = 0; a < 3; ++a)
        if (split[a] < 0 || (split[a] & 1))
            return fail(H3_ERR_INVALID_ARGUMENT, "rope_split[%d]=%d must be even and >= 0", a, split[a]);
    if (split[0] + split[1] + split[2] != head_dim)
        return fail(H3_ERR_INVALID_ARGUMENT, "rope_split sums to %d, head_dim is %d",
                    split[0] + split[1] + split[2], head_dim);
    return ok();
}

struct AttnPlan {
    int64_t items_cap;
    size_t items_bytes, bk_bytes, fp8_bytes, total;
};

AttnPlan attn_plan(int32_t num_seqs, int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                   int32_t precision) {
    AttnPlan p;
    p.items_cap = max_items(num_seqs, total_tokens, num_heads, H3_ATTN_BLOCK_M);
    p.items_bytes = align_up(static_cast<size_t>(p.items_cap) * 4 * sizeof(int32_t));
    p.bk_bytes = align_up(h3::bookkeeping_scratch_bytes(num_seqs));
    p.fp8_bytes = precision == H3_ATTN_FP8_E4M3
                      ? align_up(h3::fp8_scratch_bytes(num_seqs, total_tokens, num_heads, head_dim))
                      : 0;
    p.total = p.items_bytes + p.bk_bytes + p.fp8_bytes;
    return p;
}

h3_status check_opts(const h3_attn_opts* opts, int32_t head_dim) {
    if (opts == nullptr) return ok();
    if (opts->precision != H3_ATTN_BF16 && opts->precision != H3_ATTN_FP8_E4M3)
        return fail(H3_ERR_INVALID_ARGUMENT, "unknown attention precision %d", opts->precision);
    if (opts->precision == H3_ATTN_FP8_E4M3 && head_dim != 128)
        return fail(H3_ERR_UNSUPPORTED, "fp8 attention needs head_dim 128 (got %d)", head_dim);
    if (opts->precision == H3_ATTN_BF16 && opts->skip_softmax)
        return fail(H3_ERR_UNSUPPORTED, "skip_softmax is implemented for the fp8 path only");
    if (!(opts->softmax_scale >= 0.f) || isinf(opts->softmax_scale))
        return fail(H3_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0");
    if (isnan(opts->skip_threshold))
        return fail(H3_ERR_INVALID_ARGUMENT, "skip_threshold is NaN");
    return ok();
}

// Enqueues bookkeeping + attention; arguments already validated.
h3_status run_attention(const void* q, const void* k, const void* v, void* out, int64_t qs,
                        int64_t ks, int64_t vs, int64_t os, const int32_t* cu_dev,
                        const int32_t* cu_host, int32_t num_seqs, int32_t total_tokens,
                        int32_t num_heads, int32_t head_dim, const h3_attn_opts* opts,
                        void* workspace, hipStream_t stream) {
    const int32_t precision = opts ? opts->precision : H3_ATTN_BF16;
    const AttnPlan plan = attn_plan(num_seqs, total_tokens, num_heads, head_dim, precision);
    const int64_t n_items = count_items(cu_host, num_seqs, num_heads, H3_ATTN_BLOCK_M);
    if (n_items == 0) return ok();
    char* ws = static_cast<char*>(workspace);
    int32_t* items = reinterpret_cast<int32_t*>(ws);
    void* bk_scratch = ws + plan.items_bytes;
    void* fp8_scratch = ws + plan.items_bytes + plan.bk_bytes;
    hipError_t e = h3::launch_bookkeeping(cu_dev, num_seqs, total_tokens, num_heads,
                                          H3_ATTN_BLOCK_M, nullptr, nullptr, items,
                                          plan.items_cap, bk_scratch, stream);
    if (e != hipSuccess) return hip_fail(e, "bookkeeping launch");
    float scale = opts && opts->softmax_scale > 0.f ? opts->softmax_scale
                                                    : 1.0f / sqrtf(static_cast<float>(head_dim));
    if (precision == H3_ATTN_FP8_E4M3) {
        const float thr = opts->skip_threshold > 0.f ? opts->skip_threshold : 8.0f;
        e = h3::launch_attn_fp8(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), qs,
                                ks, vs, os, cu_dev, cu_host, items, n_items, num_seqs,
                                total_tokens, num_heads, head_dim, scale, opts->skip_softmax,
                                thr, opts->skip_counts, fp8_scratch,
                                h3::bookkeeping_rank_prefix(bk_scratch, num_seqs), stream);
        if (e != hipSuccess) return hip_fail(e, "fp8 attention launch");
        return ok();
    }
    e = h3::launch_attn_bf16(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                             static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), qs, ks,
                             vs, os, cu_dev, items, n_items, num_seqs, total_tokens, num_heads,
                             head_dim, scale, h3::bookkeeping_rank_prefix(bk_scratch, num_seqs),
                             stream);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    return ok();
}

h3_status check_gemm_shape(int64_t m, int64_t n, int64_t k, int64_t n_mult) {
    if (m < 0 || n <= 0 || k <= 0) return fail(H3_ERR_INVALID_ARGUMENT, "bad GEMM sizes m=%lld n=%lld k=%lld",
                                               (long long)m, (long long)n, (long long)k);
    if (n % n_mult) return fail(H3_ERR_UNSUPPORTED, "n=%lld must be a multiple of %lld", (long long)n, (long long)n_mult);
    if (k % 64) return fail(H3_ERR_UNSUPPORTED, "k=%lld must be a multiple of 64", (long long)k);
    if (((m + 255) / 256) * ((n + 127) / 128) > INT32_MAX / 2)
        return fail(H3_ERR_UNSUPPORTED, "m=%lld, n=%lld: too many tiles", (long long)m, (long long)n);
    return ok();
}

// Argument checks shared by h3_attn_varlen and h3_attn_varlen_noalloc (all
// but the workspace); *nothing is set when there is no work (N = 0).
h3_status check_attn_args(const void* q, const void* k, const void* v, const void* out,
                          int64_t q_tok_stride, int64_t k_tok_stride, int64_t v_tok_stride,
                          int64_t o_tok_stride, const int32_t* cu_seqlens_dev,
                          const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t total_tokens,
                          int32_t num_heads, int32_t head_dim, const h3_attn_opts* opts,
                          bool* nothing) {
    *nothing = false;
    h3_status st = check_cu(cu_seqlens_host, num_seqs, total_tokens);
    if (st != H3_OK) return st;
    if (num_heads <= 0) return fail(H3_ERR_INVALID_ARGUMENT, "num_heads=%d <= 0", num_heads);
    if (!head_dim_ok(head_dim)) return fail(H3_ERR_UNSUPPORTED, "head_dim=%d (64 or 128 only)", head_dim);
    st = check_opts(opts, head_dim);
    if (st != H3_OK) return st;
    if (total_tokens == 0) {
        *nothing = true;
        return ok();
    }
    if (!q || !k || !v || !out || !cu_seqlens_dev)
        return fail(H3_ERR_INVALID_ARGUMENT, "NULL tensor pointer");
    const int64_t row = static_cast<int64_t>(num_heads) * head_dim;
    if (q_tok_stride < row || k_tok_stride < row || v_tok_stride < row || o_tok_stride < row)
        return fail(H3_ERR_INVALID_ARGUMENT, "token strides must be >= num_heads * head_dim = %lld",
                    (long long)row);
    if ((q_tok_stride | k_tok_stride | v_tok_stride | o_tok_stride) & 7)
        return fail(H3_ERR_UNSUPPORTED, "token strides must be multiples of 8 elements");
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
         reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out)) & 15)
        return fail(H3_ERR_UNSUPPORTED, "q/k/v/out must be 16-byte aligned");
    const int32_t precision = opts ? opts->precision : H3_ATTN_BF16;
    if (opts && opts->skip_counts && precision != H3_ATTN_FP8_E4M3)
        return fail(H3_ERR_UNSUPPORTED, "skip_counts needs the fp8 path");
    return ok();
}

// ---- fixed scratch of h3_attn_varlen_noalloc ----
// One copy of the file-scope array `scratch` lives on every GPU the library
// is loaded onto, for the life of the process. In host code its name is a
// host-side stand-in, not a device address: kernels get the address
// hipGetSymbolAddress returns for the current device, looked up once per
// device (on the first call with that device current) and kept here.
constexpr size_t kNoAllocScratchBytes = H3_NOALLOC_SCRATCH_BYTES;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

h3_status noalloc_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(H3_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & (kAlign - 1)))
            return fail(H3_ERR_HIP, "scratch address %p is not 256-byte aligned", p);
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return ok();
}

}  // namespace

extern "C" {

H3_API const char* h3_status_string(h3_status status) {
    switch (status) {
        case H3_OK: return "H3_OK";
        case H3_ERR_INVALID_ARGUMENT: return "H3_ERR_INVALID_ARGUMENT";
        case H3_ERR_UNSUPPORTED: return "H3_ERR_UNSUPPORTED";
        case H3_ERR_WORKSPACE_TOO_SMALL: return "H3_ERR_WORKSPACE_TOO_SMALL";
        case H3_ERR_HIP: return "H3_ERR_HIP";
    }
    return "H3_ERR_UNKNOWN";
}

H3_API const char* h3_last_error_message(void) { return g_err; }

H3_API int32_t h3_abi_version(void) { return H3_ABI_VERSION; }

H3_API h3_status h3_build_schedule_host(const int32_t* cu_seqlens_host, int32_t num_seqs,
                                        int32_t num_heads, int32_t block_m,
                                        int32_t* items_out, int64_t capacity,
                                        int64_t* count_out) {
    if (count_out == nullptr) return fail(H3_ERR_INVALID_ARGUMENT, "count_out is NULL");
    if (num_heads <= 0) return fail(H3_ERR_INVALID_ARGUMENT, "num_heads=%d <= 0", num_heads);
    if (block_m <= 0) return fail(H3_ERR_INVALID_ARGUMENT, "block_m=%d <= 0", block_m);
    if (cu_seqlens_host == nullptr) return fail(H3_ERR_INVALID_ARGUMENT, "cu_seqlens_host is NULL");
    if (num_seqs < 0) return fail(H3_ERR_INVALID_ARGUMENT, "num_seqs < 0");
    h3_status st = check_cu(cu_seqlens_host, num_seqs, cu_seqlens_host[num_seqs]);
    if (st != H3_OK) return st;
    const int64_t count = count_items(cu_seqlens_host, num_seqs, num_heads, block_m);
    *count_out = count;
    if (items_out == nullptr) return ok();
    if (capacity < count)
        return fail(H3_ERR_WORKSPACE_TOO_SMALL, "capacity %lld < %lld items", (long long)capacity,
                    (long long)count);
    std::vector<int32_t> order(num_seqs);
    for (int32_t s = 0; s < num_seqs; ++s) order[s] = s;
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
        return (cu_seqlens_host[a + 1] - cu_seqlens_host[a]) > (cu_seqlens_host[b + 1] - cu_seqlens_host[b]);
    });
    int64_t idx = 0;
    for (int32_t s : order) {
        const int32_t len = cu_seqlens_host[s + 1] - cu_seqlens_host[s];
        for (int32_t h = 0; h < num_heads; ++h)
            for (int32_t off = 0; off < len; off += block_m) {
                int32_t* it = items_out + 4 * idx++;
                it[0] = h;
                it[1] = s;
                it[2] = cu_seqlens_host[s] + off;
                it[3] = std::min(block_m, len - off);
            }
    }
    return ok();
}

H3_API size_t h3_varlen_bookkeeping_workspace_size(int32_t num_seqs) {
    return num_seqs < 0 ? 0 : align_up(h3::bookkeeping_scratch_bytes(num_seqs));
}

H3_API h3_status h3_varlen_bookkeeping(const int32_t* cu_seqlens_dev,
                                       const int32_t* cu_seqlens_host, int32_t num_seqs,
                                       int32_t total_tokens, int32_t num_heads,
                                       int32_t block_m, int32_t* seg_id_dev,
                                       int32_t* tile_cu_dev, int32_t* items_dev,
                                       int64_t items_capacity, void* workspace,
                                       size_t workspace_bytes, void* hip_stream) {
    h3_status st = check_cu(cu_seqlens_host, num_seqs, total_tokens);
    if (st != H3_OK) return st;
    if (num_heads <= 0) return fail(H3_ERR_INVALID_ARGUMENT, "num_heads=%d <= 0", num_heads);
    if (block_m <= 0) return fail(H3_ERR_INVALID_ARGUMENT, "block_m=%d <= 0", block_m);
    if (cu_seqlens_dev == nullptr) return fail(H3_ERR_INVALID_ARGUMENT, "cu_seqlens_dev is NULL");
    const int64_t count = count_items(cu_seqlens_host, num_seqs, num_heads, block_m);
    if (items_dev != nullptr && items_capacity < count)
        return fail(H3_ERR_WORKSPACE_TOO_SMALL, "items_capacity %lld < %lld", (long long)items_capacity,
                    (long long)count);
    const size_t need = h3_varlen_bookkeeping_workspace_size(num_seqs);
    if (workspace_bytes < need || (need > 0 && workspace == nullptr))
        return fail(H3_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
    hipError_t e = h3::launch_bookkeeping(cu_seqlens_dev, num_seqs, total_tokens, num_heads,
                                          block_m, seg_id_dev, tile_cu_dev, items_dev, count,
                                          workspace, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "bookkeeping launch");
    return ok();
}

H3_API size_t h3_attn_varlen_workspace_size(int32_t num_seqs, int32_t total_tokens,
                                            int32_t num_heads, int32_t head_dim,
                                            const h3_attn_opts* opts) {
    if (num_seqs < 0 || total_tokens < 0 || num_heads <= 0 || !head_dim_ok(head_dim)) return 0;
    return attn_plan(num_seqs, total_tokens, num_heads, head_dim,
                     opts ? opts->precision : H3_ATTN_BF16).total;
}

H3_API h3_status h3_attn_varlen_num_items(const int32_t* cu_seqlens_host, int32_t num_seqs,
                                          int32_t num_heads, int64_t* count_out) {
    if (count_out == nullptr) return fail(H3_ERR_INVALID_ARGUMENT, "count_out is NULL");
    if (num_heads <= 0) return fail(H3_ERR_INVALID_ARGUMENT, "num_heads=%d <= 0", num_heads);
    if (cu_seqlens_host == nullptr || num_seqs < 0)
        return fail(H3_ERR_INVALID_ARGUMENT, "bad cu_seqlens_host / num_seqs");
    h3_status st = check_cu(cu_seqlens_host, num_seqs, cu_seqlens_host[num_seqs]);
    if (st != H3_OK) return st;
    *count_out = count_items(cu_seqlens_host, num_seqs, num_heads, H3_ATTN_BLOCK_M);
    return ok();
}

H3_API h3_status h3_attn_varlen(const void* q, const void* k, const void* v, void* out,
                                int64_t q_tok_stride, int64_t k_tok_stride,
                                int64_t v_tok_stride, int64_t o_tok_stride,
                                const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                                int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                                int32_t head_dim, const h3_attn_opts* opts, void* workspace,
                                size_t workspace_bytes, void* hip_stream) {
    bool nothing = false;
    h3_status st = check_attn_args(q, k, v, out, q_tok_stride, k_tok_stride, v_tok_stride,
                                   o_tok_stride, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                                   total_tokens, num_heads, head_dim, opts, &nothing);
    if (st != H3_OK || nothing) return st;
    const int32_t precision = opts ? opts->precision : H3_ATTN_BF16;
    const size_t need = attn_plan(num_seqs, total_tokens, num_heads, head_dim, precision).total;
    if (workspace_bytes < need || workspace == nullptr)
        return fail(H3_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))
        return fail(H3_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    return run_attention(q, k, v, out, q_tok_stride, k_tok_stride, v_tok_stride, o_tok_stride,
                         cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens, num_heads,
                         head_dim, opts, workspace, static_cast<hipStream_t>(hip_stream));
}

H3_API h3_status h3_attn_varlen_noalloc(const void* q, const void* k, const void* v, void* out,
                                        int64_t q_tok_stride, int64_t k_tok_stride,
                                        int64_t v_tok_stride, int64_t o_tok_stride,
                                        const int32_t* cu_seqlens_dev,
                                        const int32_t* cu_seqlens_host, int32_t num_seqs,
                                        int32_t total_tokens, int32_t num_heads,
                                        int32_t head_dim, const h3_attn_opts* opts,
                                        void* hip_stream) {
    bool nothing = false;
    h3_status st = check_attn_args(q, k, v, out, q_tok_stride, k_tok_stride, v_tok_stride,
                                   o_tok_stride, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                                   total_tokens, num_heads, head_dim, opts, &nothing);
    if (st != H3_OK || nothing) return st;
    const int32_t precision = opts ? opts->precision : H3_ATTN_BF16;
    const size_t need = attn_plan(num_seqs, total_tokens, num_heads, head_dim, precision).total;
    if (need > kNoAllocScratchBytes)
        return fail(H3_ERR_WORKSPACE_TOO_SMALL,
                    "h3_attn_varlen_noalloc: these sizes need %zu bytes of scratch, more than its "
                    "fixed %zu bytes; use h3_attn_varlen with a workspace", need,
                    static_cast<size_t>(kNoAllocScratchBytes));
    void* ws = nullptr;
    st = noalloc_scratch(&ws);
    if (st != H3_OK) return st;
    return run_attention(q, k, v, out, q_tok_stride, k_tok_stride, v_tok_stride, o_tok_stride,
                         cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens, num_heads,
                         head_dim, opts, ws, static_cast<hipStream_t>(hip_stream));
}

// ---- block-sparse attention, INT8 Q/K + FP8 V ----

namespace {

bool sparsity_ok(float sparsity) { return sparsity >= 0.f && sparsity < 1.f; }
int sparsity_permille(float sparsity) {
    return static_cast<int>(std::nearbyint(1000.0 * static_cast<double>(sparsity)));
}
int64_t bsa_keep(int64_t n, int permille) {
    return n > 0 ? std::max<int64_t>(1, n - (n * permille) / 1000) : 0;
}
int64_t bsa_list_stride(const int32_t* cu, int32_t num_seqs, int permille) {
    int64_t nmax = 0;
    for (int32_t s = 0; s < num_seqs; ++s)
        nmax = std::max<int64_t>(nmax, (cu[s + 1] - cu[s] + H3_FP8_QK_BLOCK - 1) / H3_FP8_QK_BLOCK);
    return std::max<int64_t>(1, bsa_keep(nmax, permille));
}
// keep(n) does not decrease with n, so the longest possible segment bounds the stride
int64_t bsa_list_stride_bound(int32_t total_tokens, int permille) {
    return std::max<int64_t>(1, bsa_keep((static_cast<int64_t>(total_tokens) + H3_FP8_QK_BLOCK - 1) /
                                             H3_FP8_QK_BLOCK, permille));
}

}  // namespace

H3_API h3_status h3_attn_block_sparse_list_stride(const int32_t* cu_seqlens_host, int32_t num_seqs,
                                                  float sparsity, int64_t* stride_out) {
    if (stride_out == nullptr) return fail(H3_ERR_INVALID_ARGUMENT, "stride_out is NULL");
    if (cu_seqlens_host == nullptr || num_seqs < 0)
        return fail(H3_ERR_INVALID_ARGUMENT, "bad cu_seqlens_host / num_seqs");
    if (!sparsity_ok(sparsity)) return fail(H3_ERR_INVALID_ARGUMENT, "sparsity must be in [0, 1)");
    h3_status st = check_cu(cu_seqlens_host, num_seqs, cu_seqlens_host[num_seqs]);
    if (st != H3_OK) return st;
    *stride_out = bsa_list_stride(cu_seqlens_host, num_seqs, sparsity_permille(sparsity));
    return ok();
}

namespace {

size_t bsa_workspace_bytes(int32_t num_seqs, int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                           float sparsity) {
    if (num_seqs < 0 || total_tokens < 0 || num_heads <= 0 || head_dim != 128 || !sparsity_ok(sparsity))
        return 0;
    const int64_t stride = bsa_list_stride_bound(total_tokens, sparsity_permille(sparsity));
    return attn_plan(num_seqs, total_tokens, num_heads, head_dim, H3_ATTN_BF16).total +
           align_up(h3::bsa_scratch_bytes(num_seqs, total_tokens, num_heads, stride));
}

// Argument checks shared by the attention entry point and the block.
h3_status check_bsa(const int32_t* cu_host, int32_t num_seqs, int32_t head_dim, float sparsity) {
    if (head_dim != 128)
        return fail(H3_ERR_UNSUPPORTED, "block-sparse attention needs head_dim 128 (got %d)", head_dim);
    if (!sparsity_ok(sparsity)) return fail(H3_ERR_INVALID_ARGUMENT, "sparsity must be in [0, 1)");
    for (int32_t s = 0; s < num_seqs; ++s)
        if (cu_host[s + 1] - cu_host[s] > h3::kBsaMaxKeyBlocks * H3_FP8_QK_BLOCK)
            return fail(H3_ERR_UNSUPPORTED, "segment %d has %d tokens; block-sparse attention takes at most %d",
                        s, cu_host[s + 1] - cu_host[s], h3::kBsaMaxKeyBlocks * H3_FP8_QK_BLOCK);
    return ok();
}

// Enqueues bookkeeping + the block-sparse pass; arguments already validated.
h3_status run_attention_bsa(const void* q, const void* k, const void* v, void* out, int64_t qs, int64_t ks,
                            int64_t vs, int64_t os, const int32_t* cu_dev, const int32_t* cu_host,
                            int32_t num_seqs, int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                            float softmax_scale, float sparsity, int32_t* lists, void* workspace,
                            hipStream_t stream) {
    const int permille = sparsity_permille(sparsity);
    const AttnPlan plan = attn_plan(num_seqs, total_tokens, num_heads, head_dim, H3_ATTN_BF16);
    const int64_t n_items = count_items(cu_host, num_seqs, num_heads, H3_ATTN_BLOCK_M);
    if (n_items == 0) return ok();
    char* ws = static_cast<char*>(workspace);
    int32_t* items = reinterpret_cast<int32_t*>(ws);
    hipError_t e = h3::launch_bookkeeping(cu_dev, num_seqs, total_tokens, num_heads, H3_ATTN_BLOCK_M,
                                          nullptr, nullptr, items, plan.items_cap, ws + plan.items_bytes,
                                          stream);
    if (e != hipSuccess) return hip_fail(e, "bookkeeping launch");
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(head_dim));
    e = h3::launch_attn_bsa(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                            static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), qs, ks, vs, os,
                            cu_dev, cu_host, items, n_items, num_seqs, total_tokens, num_heads, scale,
                            permille, bsa_list_stride(cu_host, num_seqs, permille), lists,
                            ws + plan.total, h3::bookkeeping_rank_prefix(ws + plan.items_bytes, num_seqs),
                            stream);
    if (e != hipSuccess) return hip_fail(e, "block-sparse attention launch");
    return ok();
}

}  // namespace

H3_API size_t h3_attn_block_sparse_workspace_size(int32_t num_seqs, int32_t total_tokens,
                                                  int32_t num_heads, int32_t head_dim, float sparsity) {
    return bsa_workspace_bytes(num_seqs, total_tokens, num_heads, head_dim, sparsity);
}

H3_API h3_status h3_attn_block_sparse(const void* q, const void* k, const void* v, void* out,
                                      int64_t q_tok_stride, int64_t k_tok_stride,
                                      int64_t v_tok_stride, int64_t o_tok_stride,
                                      const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                                      int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                                      int32_t head_dim, float softmax_scale, float sparsity,
                                      int32_t* kv_block_lists, void* workspace,
                                      size_t workspace_bytes, void* hip_stream) {
    h3_status st = check_cu(cu_seqlens_host, num_seqs, total_tokens);
    if (st != H3_OK) return st;
    if (num_heads <= 0) return fail(H3_ERR_INVALID_ARGUMENT, "num_heads=%d <= 0", num_heads);
    st = check_bsa(cu_seqlens_host, num_seqs, head_dim, sparsity);
    if (st != H3_OK) return st;
    if (!(softmax_scale >= 0.f) || std::isinf(softmax_scale))
        return fail(H3_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0");
    if (total_tokens == 0) return ok();
    if (!q || !k || !v || !out || !cu_seqlens_dev)
        return fail(H3_ERR_INVALID_ARGUMENT, "NULL tensor pointer");
    const int64_t row = static_cast<int64_t>(num_heads) * head_dim;
    if (q_tok_stride < row || k_tok_stride < row || v_tok_stride < row || o_tok_stride < row)
        return fail(H3_ERR_INVALID_ARGUMENT, "token strides must be >= num_heads * head_dim = %lld",
                    (long long)row);
    if ((q_tok_stride | k_tok_stride | v_tok_stride | o_tok_stride) & 7)
        return fail(H3_ERR_UNSUPPORTED, "token strides must be multiples of 8 elements");
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
         reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out)) & 15)
        return fail(H3_ERR_UNSUPPORTED, "q/k/v/out must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(kv_block_lists) & 3)
        return fail(H3_ERR_INVALID_ARGUMENT, "kv_block_lists must be 4-byte aligned");
    const size_t need = h3_attn_block_sparse_workspace_size(num_seqs, total_tokens, num_heads, head_dim, sparsity);
    if (workspace_bytes < need || workspace == nullptr)
        return fail(H3_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))
        return fail(H3_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    return run_attention_bsa(q, k, v, out, q_tok_stride, k_tok_stride, v_tok_stride, o_tok_stride,
                             cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens, num_heads, head_dim,
                             softmax_scale, sparsity, kv_block_lists, workspace,
                             static_cast<hipStream_t>(hip_stream));
}

H3_API h3_status h3_fp8_num_tiles(const int32_t* cu_seqlens_host, int32_t num_seqs,
                                  int64_t* tiles_out) {
    if (tiles_out == nullptr) return fail(H3_ERR_INVALID_ARGUMENT, "tiles_out is NULL");
    if (cu_seqlens_host == nullptr || num_seqs < 0)
        return fail(H3_ERR_INVALID_ARGUMENT, "bad cu_seqlens_host / num_seqs");
    h3_status st = check_cu(cu_seqlens_host, num_seqs, cu_seqlens_host[num_seqs]);
    if (st != H3_OK) return st;
    *tiles_out = count_items(cu_seqlens_host, num_seqs, 1, H3_FP8_QK_BLOCK);
    return ok();
}

H3_API size_t h3_fp8_quantize_workspace_size(int32_t num_seqs, int32_t total_tokens,
                                             int32_t num_heads) {
    if (num_seqs < 0 || total_tokens < 0 || num_heads <= 0) return 0;
    return align_up(h3::fp8_quant_workspace_bytes(num_seqs, total_tokens, num_heads));
}

H3_API h3_status h3_fp8_quantize(const void* q, const void* k, const void* v,
                                 int64_t q_tok_stride, int64_t k_tok_stride,
                                 int64_t v_tok_stride, const int32_t* cu_seqlens_dev,
                                 const int32_t* cu_seqlens_host, int32_t num_seqs,
                                 int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                                 void* q8, void* k8, void* v8t, float* q_scale,
                                 float* k_scale, float* v_scale, void* workspace,
                                 size_t workspace_bytes, void* hip_stream) {
    h3_status st = check_cu(cu_seqlens_host, num_seqs, total_tokens);
    if (st != H3_OK) return st;
    if (num_heads <= 0) return fail(H3_ERR_INVALID_ARGUMENT, "num_heads=%d <= 0", num_heads);
    if (head_dim != 128) return fail(H3_ERR_UNSUPPORTED, "fp8 quantisation needs head_dim 128 (got %d)", head_dim);
    if (total_tokens == 0) return ok();
    if (!q || !k || !v || !cu_seqlens_dev || !q8 || !k8 || !v8t || !q_scale || !k_scale || !v_scale)
        return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    const int64_t row = static_cast<int64_t>(num_heads) * head_dim;
    if (q_tok_stride < row || k_tok_stride < row || v_tok_stride < row)
        return fail(H3_ERR_INVALID_ARGUMENT, "token strides must be >= num_heads * head_dim = %lld",
                    (long long)row);
    if ((q_tok_stride | k_tok_stride | v_tok_stride) & 7)
        return fail(H3_ERR_UNSUPPORTED, "token strides must be multiples of 8 elements");
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
         reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(q8) |
         reinterpret_cast<uintptr_t>(k8) | reinterpret_cast<uintptr_t>(v8t)) & 15)
        return fail(H3_ERR_UNSUPPORTED, "q/k/v and the code buffers must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(q_scale) | reinterpret_cast<uintptr_t>(k_scale) |
         reinterpret_cast<uintptr_t>(v_scale)) & 3)
        return fail(H3_ERR_INVALID_ARGUMENT, "scale buffers must be 4-byte aligned");
    const size_t need = h3_fp8_quantize_workspace_size(num_seqs, total_tokens, num_heads);
    if (workspace_bytes < need || workspace == nullptr)
        return fail(H3_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))
        return fail(H3_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    const int64_t tiles = count_items(cu_seqlens_host, num_seqs, 1, H3_FP8_QK_BLOCK);
    hipError_t e = h3::launch_fp8_quantize(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
        static_cast<const uint16_t*>(v), q_tok_stride, k_tok_stride, v_tok_stride, cu_seqlens_dev,
        num_seqs, num_heads, tiles, static_cast<uint8_t*>(q8), static_cast<uint8_t*>(k8),
        static_cast<uint8_t*>(v8t), q_scale, k_scale, v_scale, workspace,
        static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "fp8 quantise launch");
    return ok();
}

H3_API h3_status h3_qk_rmsnorm_rope(void* q, void* k, int64_t q_tok_stride,
                                    int64_t k_tok_stride, const void* w_q, const void* w_k,
                                    const int32_t* rope_grid, int32_t total_tokens,
                                    int32_t num_heads, int32_t head_dim,
                                    const int32_t rope_split[3], float theta, float eps,
                                    void* hip_stream) {
    if (total_tokens < 0 || num_heads <= 0)
        return fail(H3_ERR_INVALID_ARGUMENT, "total_tokens=%d num_heads=%d", total_tokens, num_heads);
    if (!head_dim_ok(head_dim)) return fail(H3_ERR_UNSUPPORTED, "head_dim=%d (64 or 128 only)", head_dim);
    h3_status st = check_split(rope_split, head_dim);
    if (st != H3_OK) return st;
    if (!(theta > 0.f) || isinf(theta)) return fail(H3_ERR_INVALID_ARGUMENT, "theta must be finite and > 0");
    if (!(eps >= 0.f) || isinf(eps)) return fail(H3_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
    if (total_tokens == 0) return ok();
    if (!q || !k || !w_q || !w_k || !rope_grid) return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    const int64_t row = static_cast<int64_t>(num_heads) * head_dim;
    if (q_tok_stride < row || k_tok_stride < row)
        return fail(H3_ERR_INVALID_ARGUMENT, "token strides must be >= num_heads * head_dim");
    if ((q_tok_stride | k_tok_stride) & 7) return fail(H3_ERR_UNSUPPORTED, "token strides must be multiples of 8");
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
         reinterpret_cast<uintptr_t>(w_q) | reinterpret_cast<uintptr_t>(w_k)) & 15)
        return fail(H3_ERR_UNSUPPORTED, "q/k/w_q/w_k must be 16-byte aligned");
    hipError_t e = h3::launch_qk_norm_rope(static_cast<uint16_t*>(q), static_cast<uint16_t*>(k),
                                           q_tok_stride, k_tok_stride,
                                           static_cast<const uint16_t*>(w_q),
                                           static_cast<const uint16_t*>(w_k), rope_grid,
                                           total_tokens, num_heads, head_dim, rope_split, theta,
                                           eps, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "qk_rmsnorm_rope launch");
    return ok();
}

H3_API h3_status h3_modulation(const void* cond, const void* w_mod, float* mod_out,
                               int32_t num_seqs, int32_t hidden, void* hip_stream) {
    if (num_seqs < 0) return fail(H3_ERR_INVALID_ARGUMENT, "num_seqs < 0");
    if (hidden <= 0 || hidden % 512 || hidden > 8192)
        return fail(H3_ERR_UNSUPPORTED, "hidden=%d must be a multiple of 512 in [512, 8192]", hidden);
    if (num_seqs == 0) return ok();
    if (!cond || !w_mod || !mod_out) return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    if ((reinterpret_cast<uintptr_t>(cond) | reinterpret_cast<uintptr_t>(w_mod)) & 15)
        return fail(H3_ERR_UNSUPPORTED, "cond/w_mod must be 16-byte aligned");
    hipError_t e = h3::launch_modulation(static_cast<const uint16_t*>(cond),
                                         static_cast<const uint16_t*>(w_mod), mod_out, num_seqs,
                                         hidden, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "modulation launch");
    return ok();
}

H3_API h3_status h3_adaln_rmsnorm_modulate(const void* x, void* h_out, const float* shift,
                                           const float* scale, int64_t mod_row_stride,
                                           const int32_t* cu_seqlens_dev,
                                           const int32_t* cu_seqlens_host, int32_t num_seqs,
                                           int32_t total_tokens, int32_t hidden, float eps,
                                           void* hip_stream) {
    h3_status st = check_cu(cu_seqlens_host, num_seqs, total_tokens);
    if (st != H3_OK) return st;
    if (hidden <= 0 || hidden % 512 || hidden > 8192)
        return fail(H3_ERR_UNSUPPORTED, "hidden=%d must be a multiple of 512 in [512, 8192]", hidden);
    if (!(eps >= 0.f) || isinf(eps)) return fail(H3_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
    if (total_tokens == 0) return ok();
    if (!x || !h_out || !shift || !scale || !cu_seqlens_dev)
        return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (mod_row_stride < hidden || (mod_row_stride & 3))
        return fail(H3_ERR_INVALID_ARGUMENT, "mod_row_stride must be >= hidden and a multiple of 4");
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(h_out) |
         reinterpret_cast<uintptr_t>(shift) | reinterpret_cast<uintptr_t>(scale)) & 15)
        return fail(H3_ERR_UNSUPPORTED, "x/h/shift/scale must be 16-byte aligned");
    hipError_t e = h3::launch_adaln(static_cast<const uint16_t*>(x), static_cast<uint16_t*>(h_out),
                                    shift, scale, mod_row_stride, cu_seqlens_dev, num_seqs,
                                    total_tokens, hidden, eps, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "adaln launch");
    return ok();
}

H3_API h3_status h3_adaln_rmsnorm_modulate_mxfp8(const void* x, void* h_codes, void* h_scales,
                                                 const float* shift, const float* scale,
                                                 int64_t mod_row_stride,
                                                 const int32_t* cu_seqlens_dev,
                                                 const int32_t* cu_seqlens_host, int32_t num_seqs,
                                                 int32_t total_tokens, int32_t hidden, float eps,
                                                 void* hip_stream) {
    h3_status st = check_cu(cu_seqlens_host, num_seqs, total_tokens);
    if (st != H3_OK) return st;
    if (hidden <= 0 || hidden % 512 || hidden > 8192)
        return fail(H3_ERR_UNSUPPORTED, "hidden=%d must be a multiple of 512 in [512, 8192]", hidden);
    if (!(eps >= 0.f) || isinf(eps)) return fail(H3_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
    if (total_tokens == 0) return ok();
    if (!x || !h_codes || !h_scales || !shift || !scale || !cu_seqlens_dev)
        return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (mod_row_stride < hidden || (mod_row_stride & 3))
        return fail(H3_ERR_INVALID_ARGUMENT, "mod_row_stride must be >= hidden and a multiple of 4");
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(h_codes) |
         reinterpret_cast<uintptr_t>(shift) | reinterpret_cast<uintptr_t>(scale)) & 15 ||
        reinterpret_cast<uintptr_t>(h_scales) & 3)
        return fail(H3_ERR_UNSUPPORTED, "x/codes/shift/scale 16-byte and scales 4-byte aligned");
    if (static_cast<int64_t>(total_tokens) * hidden / 32 > INT32_MAX)
        return fail(H3_ERR_UNSUPPORTED, "MX scale array exceeds 2^31 bytes");
    hipError_t e = h3::launch_adaln_mx(static_cast<const uint16_t*>(x), static_cast<uint8_t*>(h_codes),
                                       static_cast<uint8_t*>(h_scales), shift, scale, mod_row_stride,
                                       cu_seqlens_dev, num_seqs, total_tokens, hidden, eps,
                                       static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "adaln launch");
    return ok();
}

H3_API h3_status h3_linear_bf16(const void* a, const void* w, void* y, int64_t m, int64_t n,
                                int64_t k, void* hip_stream) {
    h3_status st = check_gemm_shape(m, n, k, 8);
    if (st != H3_OK) return st;
    if (m == 0) return ok();
    if (!a || !w || !y) return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(w)) & 15 ||
        reinterpret_cast<uintptr_t>(y) & 7)
        return fail(H3_ERR_UNSUPPORTED, "a/w must be 16-byte and y 8-byte aligned");
    hipError_t e = h3::launch_gemm(h3::kEpiStore, static_cast<const uint16_t*>(a),
                                   static_cast<const uint16_t*>(w), nullptr,
                                   static_cast<uint16_t*>(y), m, n, k, nullptr, nullptr, 0,
                                   nullptr, 1, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "gemm launch");
    return ok();
}

H3_API h3_status h3_linear_swiglu_bf16(const void* a, const void* w_gate, const void* w_up,
                                       void* y, int64_t m, int64_t n, int64_t k,
                                       void* hip_stream) {
    h3_status st = check_gemm_shape(m, n, k, 8);
    if (st != H3_OK) return st;
    if (m == 0) return ok();
    if (!a || !w_gate || !w_up || !y) return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(w_gate) |
         reinterpret_cast<uintptr_t>(w_up)) & 15 || reinterpret_cast<uintptr_t>(y) & 7)
        return fail(H3_ERR_UNSUPPORTED, "a/w_gate/w_up must be 16-byte and y 8-byte aligned");
    hipError_t e = h3::launch_gemm(h3::kEpiSwiGLU, static_cast<const uint16_t*>(a),
                                   static_cast<const uint16_t*>(w_gate),
                                   static_cast<const uint16_t*>(w_up), static_cast<uint16_t*>(y),
                                   m, n, k, nullptr, nullptr, 0, nullptr, 1,
                                   static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "gemm launch");
    return ok();
}

H3_API h3_status h3_linear_gated_residual_bf16(const void* a, const void* w, const void* res,
                                               const float* gate, int64_t gate_row_stride,
                                               void* y, int64_t m, int64_t n, int64_t k,
                                               const int32_t* cu_seqlens_dev,
                                               const int32_t* cu_seqlens_host,
                                               int32_t num_seqs, void* hip_stream) {
    h3_status st = check_gemm_shape(m, n, k, 8);
    if (st != H3_OK) return st;
    if (m > INT32_MAX) return fail(H3_ERR_UNSUPPORTED, "m too large");
    st = check_cu(cu_seqlens_host, num_seqs, static_cast<int32_t>(m));
    if (st != H3_OK) return st;
    if (m == 0) return ok();
    if (!a || !w || !res || !gate || !y || !cu_seqlens_dev)
        return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (gate_row_stride < n) return fail(H3_ERR_INVALID_ARGUMENT, "gate_row_stride < n");
    if (gate_row_stride & 3) return fail(H3_ERR_UNSUPPORTED, "gate_row_stride must be a multiple of 4");
    if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(w) |
         reinterpret_cast<uintptr_t>(gate)) & 15 ||
        (reinterpret_cast<uintptr_t>(res) | reinterpret_cast<uintptr_t>(y)) & 7)
        return fail(H3_ERR_UNSUPPORTED, "a/w/gate must be 16-byte and res/y 8-byte aligned");
    hipError_t e = h3::launch_gemm(h3::kEpiGatedResidual, static_cast<const uint16_t*>(a),
                                   static_cast<const uint16_t*>(w), nullptr,
                                   static_cast<uint16_t*>(y), m, n, k,
                                   static_cast<const uint16_t*>(res), gate, gate_row_stride,
                                   cu_seqlens_dev, num_seqs, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "gemm launch");
    return ok();
}

H3_API h3_status h3_frames_to_uint8_bthwc(const float* x, void* out, int64_t batch, int64_t channels,
                                          int64_t frames, int64_t height, int64_t width,
                                          void* hip_stream) {
    if (batch < 0 || channels < 0 || frames < 0 || height < 0 || width < 0)
        return fail(H3_ERR_INVALID_ARGUMENT, "negative dimension");
    if (channels > 64) return fail(H3_ERR_UNSUPPORTED, "channels=%lld > 64", (long long)channels);
    if (batch == 0 || channels == 0 || frames == 0 || height == 0 || width == 0) return ok();
    const int64_t lim = static_cast<int64_t>(1) << 40;
    if (frames > lim / height || frames * height > lim / width ||
        frames * height * width > lim / (batch * channels))
        return fail(H3_ERR_UNSUPPORTED, "too many elements");
    if (!x || !out) return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (reinterpret_cast<uintptr_t>(x) & 3) return fail(H3_ERR_INVALID_ARGUMENT, "x must be 4-byte aligned");
    hipError_t e = h3::launch_frames_to_u8(x, static_cast<uint8_t*>(out), batch, static_cast<int>(channels),
                                           frames * height * width, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "frames launch");
    return ok();
}

H3_API h3_status h3_mx_quantize_bf16(const void* x, int64_t x_row_stride, int64_t rows, int64_t k,
                                     void* codes, void* scales, void* hip_stream) {
    if (rows < 0 || k <= 0) return fail(H3_ERR_INVALID_ARGUMENT, "rows=%lld k=%lld", (long long)rows, (long long)k);
    if (k % 128) return fail(H3_ERR_UNSUPPORTED, "k=%lld must be a multiple of 128", (long long)k);
    if (x_row_stride < k || x_row_stride % 8)
        return fail(H3_ERR_INVALID_ARGUMENT, "x_row_stride must be >= k and a multiple of 8");
    if (rows == 0) return ok();
    if (rows > (static_cast<int64_t>(1) << 40) / k) return fail(H3_ERR_UNSUPPORTED, "rows * k too large");
    if (!x || !codes || !scales) return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(codes)) & 15 ||
        reinterpret_cast<uintptr_t>(scales) & 3)
        return fail(H3_ERR_UNSUPPORTED, "x and codes must be 16-byte, scales 4-byte aligned");
    hipError_t e = h3::launch_mx_quantize(static_cast<const uint16_t*>(x), x_row_stride, rows, k,
                                          static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales),
                                          static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "mx quantize launch");
    return ok();
}

}  // extern "C"

namespace {

// MX GEMM operands: k a multiple of 128, codes 16-byte and scales 4-byte
// aligned, and every scale array's byte count within a signed 32-bit range
// (the kernel addresses it with 32-bit buffer offsets).
h3_status check_mx_gemm(int64_t m, int64_t n, int64_t k, int64_t n_mult) {
    h3_status st = check_gemm_shape(m, n, k, n_mult);
    if (st != H3_OK) return st;
    if (k % 128) return fail(H3_ERR_UNSUPPORTED, "k=%lld must be a multiple of 128 (MX)", (long long)k);
    if (std::max(m, n) > INT32_MAX / (k / 32))
        return fail(H3_ERR_UNSUPPORTED, "m or n times k/32 exceeds 2^31 (MX scale arrays)");
    return ok();
}

bool mx_aligned(const void* codes, const void* scales) {
    return !((reinterpret_cast<uintptr_t>(codes) & 15) || (reinterpret_cast<uintptr_t>(scales) & 3));
}

}  // namespace

extern "C" {

H3_API h3_status h3_linear_mxfp8(const void* a, const void* a_scales, const void* w,
                                 const void* w_scales, void* y, int64_t m, int64_t n, int64_t k,
                                 void* hip_stream) {
    h3_status st = check_mx_gemm(m, n, k, 8);
    if (st != H3_OK) return st;
    if (m == 0) return ok();
    if (!a || !a_scales || !w || !w_scales || !y) return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (!mx_aligned(a, a_scales) || !mx_aligned(w, w_scales) || reinterpret_cast<uintptr_t>(y) & 7)
        return fail(H3_ERR_UNSUPPORTED, "codes 16-byte, scales 4-byte and y 8-byte aligned");
    hipError_t e = h3::launch_gemm_mx(h3::kEpiStore, static_cast<const uint8_t*>(a),
                                      static_cast<const uint8_t*>(a_scales), static_cast<const uint8_t*>(w),
                                      static_cast<const uint8_t*>(w_scales), nullptr, nullptr, y, nullptr,
                                      m, n, k, nullptr, nullptr, 0, nullptr, 1,
                                      static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "mx gemm launch");
    return ok();
}

H3_API h3_status h3_linear_swiglu_mxfp8(const void* a, const void* a_scales, const void* w_gate,
                                        const void* w_gate_scales, const void* w_up,
                                        const void* w_up_scales, void* y, void* y_scales, int64_t m,
                                        int64_t n, int64_t k, void* hip_stream) {
    h3_status st = check_mx_gemm(m, n, k, 128);
    if (st != H3_OK) return st;
    if (m == 0) return ok();
    if (!a || !a_scales || !w_gate || !w_gate_scales || !w_up || !w_up_scales || !y || !y_scales)
        return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (m > INT32_MAX / (n / 32)) return fail(H3_ERR_UNSUPPORTED, "m * n / 32 exceeds 2^31");
    if (!mx_aligned(a, a_scales) || !mx_aligned(w_gate, w_gate_scales) || !mx_aligned(w_up, w_up_scales) ||
        !mx_aligned(y, y_scales))
        return fail(H3_ERR_UNSUPPORTED, "codes 16-byte and scales 4-byte aligned");
    hipError_t e = h3::launch_gemm_mx(h3::kEpiSwiGLU, static_cast<const uint8_t*>(a),
                                      static_cast<const uint8_t*>(a_scales), static_cast<const uint8_t*>(w_gate),
                                      static_cast<const uint8_t*>(w_gate_scales),
                                      static_cast<const uint8_t*>(w_up), static_cast<const uint8_t*>(w_up_scales),
                                      y, static_cast<uint8_t*>(y_scales), m, n, k, nullptr, nullptr, 0,
                                      nullptr, 1, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "mx gemm launch");
    return ok();
}

H3_API h3_status h3_linear_gated_residual_mxfp8(const void* a, const void* a_scales, const void* w,
                                                const void* w_scales, const void* res,
                                                const float* gate, int64_t gate_row_stride, void* y,
                                                int64_t m, int64_t n, int64_t k,
                                                const int32_t* cu_seqlens_dev,
                                                const int32_t* cu_seqlens_host, int32_t num_seqs,
                                                void* hip_stream) {
    h3_status st = check_mx_gemm(m, n, k, 8);
    if (st != H3_OK) return st;
    if (m > INT32_MAX) return fail(H3_ERR_UNSUPPORTED, "m too large");
    st = check_cu(cu_seqlens_host, num_seqs, static_cast<int32_t>(m));
    if (st != H3_OK) return st;
    if (m == 0) return ok();
    if (!a || !a_scales || !w || !w_scales || !res || !gate || !y || !cu_seqlens_dev)
        return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (gate_row_stride < n) return fail(H3_ERR_INVALID_ARGUMENT, "gate_row_stride < n");
    if (gate_row_stride & 3) return fail(H3_ERR_UNSUPPORTED, "gate_row_stride must be a multiple of 4");
    if (!mx_aligned(a, a_scales) || !mx_aligned(w, w_scales) || reinterpret_cast<uintptr_t>(gate) & 15 ||
        (reinterpret_cast<uintptr_t>(res) | reinterpret_cast<uintptr_t>(y)) & 7)
        return fail(H3_ERR_UNSUPPORTED, "codes/gate 16-byte, scales 4-byte, res/y 8-byte aligned");
    hipError_t e = h3::launch_gemm_mx(h3::kEpiGatedResidual, static_cast<const uint8_t*>(a),
                                      static_cast<const uint8_t*>(a_scales), static_cast<const uint8_t*>(w),
                                      static_cast<const uint8_t*>(w_scales), nullptr, nullptr, y, nullptr,
                                      m, n, k, static_cast<const uint16_t*>(res), gate, gate_row_stride,
                                      cu_seqlens_dev, num_seqs, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "mx gemm launch");
    return ok();
}

}  // extern "C"

namespace {

// MXFP4 GEMM operands: k a multiple of 256 (one K step of 128 bytes per row),
// codes 16-byte and scales 8-byte aligned, scale arrays within 2^31 bytes.
h3_status check_mx4_gemm(int64_t m, int64_t n, int64_t k, int64_t n_mult) {
    h3_status st = check_gemm_shape(m, n, k, n_mult);
    if (st != H3_OK) return st;
    if (k % 256) return fail(H3_ERR_UNSUPPORTED, "k=%lld must be a multiple of 256 (MXFP4)", (long long)k);
    if (std::max(m, n) > INT32_MAX / (k / 32))
        return fail(H3_ERR_UNSUPPORTED, "m or n times k/32 exceeds 2^31 (MX scale arrays)");
    return ok();
}

bool mx4_aligned(const void* codes, const void* scales) {
    return !((reinterpret_cast<uintptr_t>(codes) & 15) || (reinterpret_cast<uintptr_t>(scales) & 7));
}

}  // namespace

extern "C" {

H3_API h3_status h3_mx4_quantize_bf16(const void* x, int64_t x_row_stride, int64_t rows, int64_t k,
                                      void* codes, void* scales, void* hip_stream) {
    if (rows < 0 || k <= 0) return fail(H3_ERR_INVALID_ARGUMENT, "rows=%lld k=%lld", (long long)rows, (long long)k);
    if (k % 256) return fail(H3_ERR_UNSUPPORTED, "k=%lld must be a multiple of 256", (long long)k);
    if (x_row_stride < k || x_row_stride % 8)
        return fail(H3_ERR_INVALID_ARGUMENT, "x_row_stride must be >= k and a multiple of 8");
    if (rows == 0) return ok();
    if (rows > (static_cast<int64_t>(1) << 40) / k) return fail(H3_ERR_UNSUPPORTED, "rows * k too large");
    if (!x || !codes || !scales) return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(codes)) & 15 ||
        reinterpret_cast<uintptr_t>(scales) & 7)
        return fail(H3_ERR_UNSUPPORTED, "x and codes must be 16-byte, scales 8-byte aligned");
    hipError_t e = h3::launch_mx4_quantize(static_cast<const uint16_t*>(x), x_row_stride, rows, k,
                                           static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales),
                                           static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "mxfp4 quantize launch");
    return ok();
}

H3_API h3_status h3_linear_mxfp4(const void* a, const void* a_scales, const void* w,
                                 const void* w_scales, void* y, int64_t m, int64_t n, int64_t k,
                                 void* hip_stream) {
    h3_status st = check_mx4_gemm(m, n, k, 8);
    if (st != H3_OK) return st;
    if (m == 0) return ok();
    if (!a || !a_scales || !w || !w_scales || !y) return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (!mx4_aligned(a, a_scales) || !mx4_aligned(w, w_scales) || reinterpret_cast<uintptr_t>(y) & 7)
        return fail(H3_ERR_UNSUPPORTED, "codes 16-byte, scales 8-byte and y 8-byte aligned");
    hipError_t e = h3::launch_gemm_mx4(h3::kEpiStore, static_cast<const uint8_t*>(a),
                                       static_cast<const uint8_t*>(a_scales), static_cast<const uint8_t*>(w),
                                       static_cast<const uint8_t*>(w_scales), nullptr, nullptr, y, m, n, k,
                                       nullptr, nullptr, 0, nullptr, 1, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "mxfp4 gemm launch");
    return ok();
}

H3_API h3_status h3_linear_swiglu_mxfp4(const void* a, const void* a_scales, const void* w_gate,
                                        const void* w_gate_scales, const void* w_up,
                                        const void* w_up_scales, void* y, int64_t m, int64_t n,
                                        int64_t k, void* hip_stream) {
    h3_status st = check_mx4_gemm(m, n, k, 128);
    if (st != H3_OK) return st;
    if (m == 0) return ok();
    if (!a || !a_scales || !w_gate || !w_gate_scales || !w_up || !w_up_scales || !y)
        return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (!mx4_aligned(a, a_scales) || !mx4_aligned(w_gate, w_gate_scales) || !mx4_aligned(w_up, w_up_scales) ||
        reinterpret_cast<uintptr_t>(y) & 7)
        return fail(H3_ERR_UNSUPPORTED, "codes 16-byte, scales 8-byte and y 8-byte aligned");
    hipError_t e = h3::launch_gemm_mx4(h3::kEpiSwiGLU, static_cast<const uint8_t*>(a),
                                       static_cast<const uint8_t*>(a_scales), static_cast<const uint8_t*>(w_gate),
                                       static_cast<const uint8_t*>(w_gate_scales),
                                       static_cast<const uint8_t*>(w_up), static_cast<const uint8_t*>(w_up_scales),
                                       y, m, n, k, nullptr, nullptr, 0, nullptr, 1,
                                       static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "mxfp4 gemm launch");
    return ok();
}

H3_API h3_status h3_linear_gated_residual_mxfp4(const void* a, const void* a_scales, const void* w,
                                                const void* w_scales, const void* res,
                                                const float* gate, int64_t gate_row_stride, void* y,
                                                int64_t m, int64_t n, int64_t k,
                                                const int32_t* cu_seqlens_dev,
                                                const int32_t* cu_seqlens_host, int32_t num_seqs,
                                                void* hip_stream) {
    h3_status st = check_mx4_gemm(m, n, k, 8);
    if (st != H3_OK) return st;
    if (m > INT32_MAX) return fail(H3_ERR_UNSUPPORTED, "m too large");
    st = check_cu(cu_seqlens_host, num_seqs, static_cast<int32_t>(m));
    if (st != H3_OK) return st;
    if (m == 0) return ok();
    if (!a || !a_scales || !w || !w_scales || !res || !gate || !y || !cu_seqlens_dev)
        return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (gate_row_stride < n) return fail(H3_ERR_INVALID_ARGUMENT, "gate_row_stride < n");
    if (gate_row_stride & 3) return fail(H3_ERR_UNSUPPORTED, "gate_row_stride must be a multiple of 4");
    if (!mx4_aligned(a, a_scales) || !mx4_aligned(w, w_scales) || reinterpret_cast<uintptr_t>(gate) & 15 ||
        (reinterpret_cast<uintptr_t>(res) | reinterpret_cast<uintptr_t>(y)) & 7)
        return fail(H3_ERR_UNSUPPORTED, "codes/gate 16-byte, scales 8-byte, res/y 8-byte aligned");
    hipError_t e = h3::launch_gemm_mx4(h3::kEpiGatedResidual, static_cast<const uint8_t*>(a),
                                       static_cast<const uint8_t*>(a_scales), static_cast<const uint8_t*>(w),
                                       static_cast<const uint8_t*>(w_scales), nullptr, nullptr, y, m, n, k,
                                       static_cast<const uint16_t*>(res), gate, gate_row_stride,
                                       cu_seqlens_dev, num_seqs, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "mxfp4 gemm launch");
    return ok();
}

}  // extern "C"

namespace {

struct BlockPlan {
    size_t mod, h, qkv, o, x1, h2, a, attn, total;
};

BlockPlan block_plan(const h3_dit_dims* d, int32_t num_seqs, int32_t total_tokens) {
    BlockPlan p;
    const size_t n = static_cast<size_t>(total_tokens), c = static_cast<size_t>(d->hidden);
    p.mod = align_up(static_cast<size_t>(num_seqs) * 6 * c * sizeof(float));
    p.h = align_up(n * c * 2);
    p.qkv = align_up(n * 3 * c * 2);
    p.o = p.h;
    p.x1 = p.h;
    p.h2 = p.h;
    p.a = align_up(n * static_cast<size_t>(d->ffn_dim) * 2);
    p.attn = attn_plan(num_seqs, total_tokens, d->num_heads, d->head_dim, H3_ATTN_BF16).total;
    p.total = p.mod + p.h + p.qkv + p.o + p.x1 + p.h2 + p.a + p.attn;
    return p;
}

h3_status check_dims(const h3_dit_dims* d) {
    if (d == nullptr) return fail(H3_ERR_INVALID_ARGUMENT, "dims is NULL");
    if (d->num_heads <= 0 || d->head_dim <= 0 || d->hidden <= 0 || d->ffn_dim <= 0)
        return fail(H3_ERR_INVALID_ARGUMENT, "dims must be positive");
    if (!head_dim_ok(d->head_dim)) return fail(H3_ERR_UNSUPPORTED, "head_dim=%d (64 or 128 only)", d->head_dim);
    if (static_cast<int64_t>(d->num_heads) * d->head_dim != d->hidden)
        return fail(H3_ERR_INVALID_ARGUMENT, "hidden=%d != num_heads*head_dim=%d", d->hidden,
                    d->num_heads * d->head_dim);
    if (d->hidden % 512 || d->hidden > 8192)
        return fail(H3_ERR_UNSUPPORTED, "hidden=%d must be a multiple of 512 up to 8192", d->hidden);
    if (d->ffn_dim % 64) return fail(H3_ERR_UNSUPPORTED, "ffn_dim=%d must be a multiple of 64", d->ffn_dim);
    h3_status st = check_split(d->rope_split, d->head_dim);
    if (st != H3_OK) return st;
    if (!(d->rope_theta > 0.f) || isinf(d->rope_theta))
        return fail(H3_ERR_INVALID_ARGUMENT, "rope_theta must be finite and > 0");
    if (!(d->eps >= 0.f) || isinf(d->eps)) return fail(H3_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
    return ok();
}

}  // namespace

extern "C" {

H3_API size_t h3_dit_block_workspace_size(const h3_dit_dims* dims, int32_t num_seqs,
                                          int32_t total_tokens) {
    if (dims == nullptr || num_seqs < 0 || total_tokens < 0) return 0;
    if (check_dims(dims) != H3_OK) return 0;
    return block_plan(dims, num_seqs, total_tokens).total;
}

H3_API h3_status h3_dit_block_forward(const void* x, void* x_out, const void* cond,
                                      const h3_dit_weights* weights, const h3_dit_dims* dims,
                                      const int32_t* cu_seqlens_dev,
                                      const int32_t* cu_seqlens_host, int32_t num_seqs,
                                      int32_t total_tokens, const int32_t* rope_grid,
                                      const h3_dit_taps* taps, void* workspace,
                                      size_t workspace_bytes, void* hip_stream) {
    h3_status st = check_dims(dims);
    if (st != H3_OK) return st;
    st = check_cu(cu_seqlens_host, num_seqs, total_tokens);
    if (st != H3_OK) return st;
    if (total_tokens == 0) return ok();
    if (!x || !x_out || !cond || !weights || !cu_seqlens_dev || !rope_grid)
        return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    const h3_dit_weights& w = *weights;
    if (!w.w_mod || !w.w_qkv || !w.w_o || !w.q_norm || !w.k_norm || !w.w_gate || !w.w_up || !w.w_down)
        return fail(H3_ERR_INVALID_ARGUMENT, "NULL weight pointer");
    if (x == x_out) return fail(H3_ERR_INVALID_ARGUMENT, "x and x_out may not alias");
    const uintptr_t al = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(x_out) |
                         reinterpret_cast<uintptr_t>(cond) | reinterpret_cast<uintptr_t>(w.w_mod) |
                         reinterpret_cast<uintptr_t>(w.w_qkv) | reinterpret_cast<uintptr_t>(w.w_o) |
                         reinterpret_cast<uintptr_t>(w.q_norm) | reinterpret_cast<uintptr_t>(w.k_norm) |
                         reinterpret_cast<uintptr_t>(w.w_gate) | reinterpret_cast<uintptr_t>(w.w_up) |
                         reinterpret_cast<uintptr_t>(w.w_down);
    if (al & 15) return fail(H3_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
    const BlockPlan p = block_plan(dims, num_seqs, total_tokens);
    if (workspace_bytes < p.total || workspace == nullptr)
        return fail(H3_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, p.total);
    if (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))
        return fail(H3_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    if (taps) {
        const uintptr_t t = reinterpret_cast<uintptr_t>(taps->mod) | reinterpret_cast<uintptr_t>(taps->h) |
                            reinterpret_cast<uintptr_t>(taps->qkv) | reinterpret_cast<uintptr_t>(taps->o) |
                            reinterpret_cast<uintptr_t>(taps->x1) | reinterpret_cast<uintptr_t>(taps->h2) |
                            reinterpret_cast<uintptr_t>(taps->a);
        if (t & 15) return fail(H3_ERR_UNSUPPORTED, "tap buffers must be 16-byte aligned");
    }

    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    char* ws = static_cast<char*>(workspace);
    auto carve = [&](size_t bytes) { char* r = ws; ws += bytes; return r; };
    float* mod = reinterpret_cast<float*>(carve(p.mod));
    uint16_t* hbuf = reinterpret_cast<uint16_t*>(carve(p.h));
    uint16_t* qkv = reinterpret_cast<uint16_t*>(carve(p.qkv));
    uint16_t* obuf = reinterpret_cast<uint16_t*>(carve(p.o));
    uint16_t* x1 = reinterpret_cast<uint16_t*>(carve(p.x1));
    uint16_t* h2 = reinterpret_cast<uint16_t*>(carve(p.h2));
    uint16_t* abuf = reinterpret_cast<uint16_t*>(carve(p.a));
    void* attn_ws = carve(p.attn);
    if (taps) {
        if (taps->mod) mod = taps->mod;
        if (taps->h) hbuf = static_cast<uint16_t*>(taps->h);
        if (taps->qkv) qkv = static_cast<uint16_t*>(taps->qkv);
        if (taps->o) obuf = static_cast<uint16_t*>(taps->o);
        if (taps->x1) x1 = static_cast<uint16_t*>(taps->x1);
        if (taps->h2) h2 = static_cast<uint16_t*>(taps->h2);
        if (taps->a) abuf = static_cast<uint16_t*>(taps->a);
    }

    const int64_t n = total_tokens, c = dims->hidden, ffn = dims->ffn_dim;
    const int64_t ms = 6 * c;
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    uint16_t* yb = static_cast<uint16_t*>(x_out);
    hipError_t e;
#define H3_TRY(call, what)                          \
    e = (call);                                     \
    if (e != hipSuccess) return hip_fail(e, what);

    H3_TRY(h3::launch_modulation(static_cast<const uint16_t*>(cond),
                                 static_cast<const uint16_t*>(w.w_mod), mod, num_seqs,
                                 static_cast<int>(c), stream), "modulation");
    H3_TRY(h3::launch_adaln(xb, hbuf, mod + 0 * c, mod + 1 * c, ms, cu_seqlens_dev, num_seqs,
                            total_tokens, static_cast<int>(c), dims->eps, stream), "adaln 1");
    H3_TRY(h3::launch_gemm(h3::kEpiStore, hbuf, static_cast<const uint16_t*>(w.w_qkv), nullptr,
                           qkv, n, 3 * c, c, nullptr, nullptr, 0, nullptr, 1, stream), "qkv gemm");
    H3_TRY(h3::launch_qk_norm_rope(qkv, qkv + c, 3 * c, 3 * c,
                                   static_cast<const uint16_t*>(w.q_norm),
                                   static_cast<const uint16_t*>(w.k_norm), rope_grid,
                                   total_tokens, dims->num_heads, dims->head_dim,
                                   dims->rope_split, dims->rope_theta, dims->eps, stream),
           "qk norm rope");
    h3_status ast = run_attention(qkv, qkv + c, qkv + 2 * c, obuf, 3 * c, 3 * c, 3 * c, c,
                                  cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens,
                                  dims->num_heads, dims->head_dim, nullptr, attn_ws, stream);
    if (ast != H3_OK) return ast;
    H3_TRY(h3::launch_gemm(h3::kEpiGatedResidual, obuf, static_cast<const uint16_t*>(w.w_o),
                           nullptr, x1, n, c, c, xb, mod + 2 * c, ms, cu_seqlens_dev, num_seqs,
                           stream), "out-proj gemm");
    H3_TRY(h3::launch_adaln(x1, h2, mod + 3 * c, mod + 4 * c, ms, cu_seqlens_dev, num_seqs,
                            total_tokens, static_cast<int>(c), dims->eps, stream), "adaln 2");
    H3_TRY(h3::launch_gemm(h3::kEpiSwiGLU, h2, static_cast<const uint16_t*>(w.w_gate),
                           static_cast<const uint16_t*>(w.w_up), abuf, n, ffn, c, nullptr,
                           nullptr, 0, nullptr, 1, stream), "gate/up gemm");
    H3_TRY(h3::launch_gemm(h3::kEpiGatedResidual, abuf, static_cast<const uint16_t*>(w.w_down),
                           nullptr, yb, n, c, ffn, x1, mod + 5 * c, ms, cu_seqlens_dev,
                           num_seqs, stream), "down gemm");
#undef H3_TRY
    return ok();
}

}  // extern "C"

namespace {

struct BlockPlanMX {
    size_t mod, h8, hs, qkv, o, o8, os, x1, a8, as, attn, total;
};

// sparsity < 0: dense bf16 attention; else block-sparse at that sparsity
BlockPlanMX block_plan_mx(const h3_dit_dims* d, int32_t num_seqs, int32_t total_tokens,
                          float sparsity = -1.f) {
    BlockPlanMX p;
    const size_t n = static_cast<size_t>(total_tokens), c = static_cast<size_t>(d->hidden);
    const size_t f = static_cast<size_t>(d->ffn_dim);
    p.mod = align_up(static_cast<size_t>(num_seqs) * 6 * c * sizeof(float));
    p.h8 = align_up(n * c);              // h, then h2 (MX codes)
    p.hs = align_up(n * c / 32);
    p.qkv = align_up(n * 3 * c * 2);
    p.o = align_up(n * c * 2);
    p.o8 = align_up(n * c);
    p.os = align_up(n * c / 32);
    p.x1 = align_up(n * c * 2);
    p.a8 = align_up(n * f);
    p.as = align_up(n * f / 32);
    p.attn = sparsity < 0.f ? attn_plan(num_seqs, total_tokens, d->num_heads, d->head_dim, H3_ATTN_BF16).total
                            : bsa_workspace_bytes(num_seqs, total_tokens, d->num_heads, d->head_dim, sparsity);
    p.total = p.mod + p.h8 + p.hs + p.qkv + p.o + p.o8 + p.os + p.x1 + p.a8 + p.as + p.attn;
    return p;
}

h3_status check_dims_mx(const h3_dit_dims* d, int32_t total_tokens) {
    h3_status st = check_dims(d);
    if (st != H3_OK) return st;
    if (d->ffn_dim % 128) return fail(H3_ERR_UNSUPPORTED, "ffn_dim=%d must be a multiple of 128 (MX)", d->ffn_dim);
    const int64_t widest = std::max<int64_t>(3 * static_cast<int64_t>(d->hidden), d->ffn_dim);
    if (static_cast<int64_t>(total_tokens) * widest / 32 > INT32_MAX ||
        widest * std::max(d->hidden, d->ffn_dim) / 32 > INT32_MAX)
        return fail(H3_ERR_UNSUPPORTED, "MX scale arrays exceed 2^31 bytes");
    return ok();
}

}  // namespace

extern "C" {

H3_API size_t h3_dit_block_mx_workspace_size(const h3_dit_dims* dims, int32_t num_seqs,
                                             int32_t total_tokens) {
    if (dims == nullptr || num_seqs < 0 || total_tokens < 0) return 0;
    if (check_dims_mx(dims, total_tokens) != H3_OK) return 0;
    return block_plan_mx(dims, num_seqs, total_tokens).total;
}

}  // extern "C"

namespace {

// The MXFP8 block; sparsity < 0 runs dense bf16 attention, otherwise the
// block-sparse INT8/FP8 attention at that sparsity.
h3_status block_forward_mx(const void* x, void* x_out, const void* cond, const h3_dit_mx_weights* weights,
                           const h3_dit_dims* dims, const int32_t* cu_seqlens_dev,
                           const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t total_tokens,
                           const int32_t* rope_grid, float sparsity, void* workspace,
                           size_t workspace_bytes, void* hip_stream) {
    h3_status st = check_dims_mx(dims, total_tokens);
    if (st != H3_OK) return st;
    st = check_cu(cu_seqlens_host, num_seqs, total_tokens);
    if (st != H3_OK) return st;
    if (sparsity >= 0.f) {
        st = check_bsa(cu_seqlens_host, num_seqs, dims->head_dim, sparsity);
        if (st != H3_OK) return st;
    }
    if (total_tokens == 0) return ok();
    if (!x || !x_out || !cond || !weights || !cu_seqlens_dev || !rope_grid)
        return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    const h3_dit_mx_weights& w = *weights;
    const h3_mx_matrix* mats[5] = {&w.w_qkv, &w.w_o, &w.w_gate, &w.w_up, &w.w_down};
    if (!w.w_mod || !w.q_norm || !w.k_norm) return fail(H3_ERR_INVALID_ARGUMENT, "NULL weight pointer");
    for (const h3_mx_matrix* m : mats) {
        if (!m->codes || !m->scales) return fail(H3_ERR_INVALID_ARGUMENT, "NULL MX weight pointer");
        if (!mx_aligned(m->codes, m->scales))
            return fail(H3_ERR_UNSUPPORTED, "MX weight codes 16-byte and scales 4-byte aligned");
    }
    if (x == x_out) return fail(H3_ERR_INVALID_ARGUMENT, "x and x_out may not alias");
    const uintptr_t al = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(x_out) |
                         reinterpret_cast<uintptr_t>(cond) | reinterpret_cast<uintptr_t>(w.w_mod) |
                         reinterpret_cast<uintptr_t>(w.q_norm) | reinterpret_cast<uintptr_t>(w.k_norm);
    if (al & 15) return fail(H3_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
    const BlockPlanMX p = block_plan_mx(dims, num_seqs, total_tokens, sparsity);
    if (workspace_bytes < p.total || workspace == nullptr)
        return fail(H3_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, p.total);
    if (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))
        return fail(H3_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");

    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    char* ws = static_cast<char*>(workspace);
    auto carve = [&](size_t bytes) { char* r = ws; ws += bytes; return r; };
    float* mod = reinterpret_cast<float*>(carve(p.mod));
    uint8_t* h8 = reinterpret_cast<uint8_t*>(carve(p.h8));
    uint8_t* hs = reinterpret_cast<uint8_t*>(carve(p.hs));
    uint16_t* qkv = reinterpret_cast<uint16_t*>(carve(p.qkv));
    uint16_t* obuf = reinterpret_cast<uint16_t*>(carve(p.o));
    uint8_t* o8 = reinterpret_cast<uint8_t*>(carve(p.o8));
    uint8_t* os = reinterpret_cast<uint8_t*>(carve(p.os));
    uint16_t* x1 = reinterpret_cast<uint16_t*>(carve(p.x1));
    uint8_t* a8 = reinterpret_cast<uint8_t*>(carve(p.a8));
    uint8_t* as = reinterpret_cast<uint8_t*>(carve(p.as));
    void* attn_ws = carve(p.attn);

    const int64_t n = total_tokens, c = dims->hidden, ffn = dims->ffn_dim;
    const int64_t ms = 6 * c;
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    uint16_t* yb = static_cast<uint16_t*>(x_out);
    auto u8 = [](const void* ptr) { return static_cast<const uint8_t*>(ptr); };
    hipError_t e;
#define H3_TRY(call, what)                          \
    e = (call);                                     \
    if (e != hipSuccess) return hip_fail(e, what);

    H3_TRY(h3::launch_modulation(static_cast<const uint16_t*>(cond),
                                 static_cast<const uint16_t*>(w.w_mod), mod, num_seqs,
                                 static_cast<int>(c), stream), "modulation");
    H3_TRY(h3::launch_adaln_mx(xb, h8, hs, mod + 0 * c, mod + 1 * c, ms, cu_seqlens_dev, num_seqs,
                               total_tokens, static_cast<int>(c), dims->eps, stream), "adaln 1");
    H3_TRY(h3::launch_gemm_mx(h3::kEpiStore, h8, hs, u8(w.w_qkv.codes), u8(w.w_qkv.scales), nullptr,
                              nullptr, qkv, nullptr, n, 3 * c, c, nullptr, nullptr, 0, nullptr, 1,
                              stream), "qkv gemm");
    H3_TRY(h3::launch_qk_norm_rope(qkv, qkv + c, 3 * c, 3 * c,
                                   static_cast<const uint16_t*>(w.q_norm),
                                   static_cast<const uint16_t*>(w.k_norm), rope_grid,
                                   total_tokens, dims->num_heads, dims->head_dim,
                                   dims->rope_split, dims->rope_theta, dims->eps, stream),
           "qk norm rope");
    h3_status ast = sparsity < 0.f
                        ? run_attention(qkv, qkv + c, qkv + 2 * c, obuf, 3 * c, 3 * c, 3 * c, c,
                                        cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens,
                                        dims->num_heads, dims->head_dim, nullptr, attn_ws, stream)
                        : run_attention_bsa(qkv, qkv + c, qkv + 2 * c, obuf, 3 * c, 3 * c, 3 * c, c,
                                            cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens,
                                            dims->num_heads, dims->head_dim, 0.f, sparsity, nullptr,
                                            attn_ws, stream);
    if (ast != H3_OK) return ast;
    H3_TRY(h3::launch_mx_quantize(obuf, c, n, c, o8, os, stream), "o quantize");
    H3_TRY(h3::launch_gemm_mx(h3::kEpiGatedResidual, o8, os, u8(w.w_o.codes), u8(w.w_o.scales), nullptr,
                              nullptr, x1, nullptr, n, c, c, xb, mod + 2 * c, ms, cu_seqlens_dev,
                              num_seqs, stream), "out-proj gemm");
    H3_TRY(h3::launch_adaln_mx(x1, h8, hs, mod + 3 * c, mod + 4 * c, ms, cu_seqlens_dev, num_seqs,
                               total_tokens, static_cast<int>(c), dims->eps, stream), "adaln 2");
    H3_TRY(h3::launch_gemm_mx(h3::kEpiSwiGLU, h8, hs, u8(w.w_gate.codes), u8(w.w_gate.scales),
                              u8(w.w_up.codes), u8(w.w_up.scales), a8, as, n, ffn, c, nullptr,
                              nullptr, 0, nullptr, 1, stream), "gate/up gemm");
    H3_TRY(h3::launch_gemm_mx(h3::kEpiGatedResidual, a8, as, u8(w.w_down.codes), u8(w.w_down.scales),
                              nullptr, nullptr, yb, nullptr, n, c, ffn, x1, mod + 5 * c, ms,
                              cu_seqlens_dev, num_seqs, stream), "down gemm");
#undef H3_TRY
    return ok();
}

}  // namespace

extern "C" {

H3_API h3_status h3_dit_block_forward_mxfp8(const void* x, void* x_out, const void* cond,
                                            const h3_dit_mx_weights* weights,
                                            const h3_dit_dims* dims,
                                            const int32_t* cu_seqlens_dev,
                                            const int32_t* cu_seqlens_host, int32_t num_seqs,
                                            int32_t total_tokens, const int32_t* rope_grid,
                                            void* workspace, size_t workspace_bytes,
                                            void* hip_stream) {
    return block_forward_mx(x, x_out, cond, weights, dims, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                            total_tokens, rope_grid, -1.f, workspace, workspace_bytes, hip_stream);
}

H3_API size_t h3_dit_block_mx_bsa_workspace_size(const h3_dit_dims* dims, int32_t num_seqs,
                                                 int32_t total_tokens, float sparsity) {
    if (dims == nullptr || num_seqs < 0 || total_tokens < 0 || !sparsity_ok(sparsity)) return 0;
    if (check_dims_mx(dims, total_tokens) != H3_OK || dims->head_dim != 128) return 0;
    return block_plan_mx(dims, num_seqs, total_tokens, sparsity).total;
}

H3_API h3_status h3_dit_block_forward_mxfp8_bsa(const void* x, void* x_out, const void* cond,
                                                const h3_dit_mx_weights* weights,
                                                const h3_dit_dims* dims,
                                                const int32_t* cu_seqlens_dev,
                                                const int32_t* cu_seqlens_host, int32_t num_seqs,
                                                int32_t total_tokens, const int32_t* rope_grid,
                                                float sparsity, void* workspace,
                                                size_t workspace_bytes, void* hip_stream) {
    if (!sparsity_ok(sparsity)) return fail(H3_ERR_INVALID_ARGUMENT, "sparsity must be in [0, 1)");
    return block_forward_mx(x, x_out, cond, weights, dims, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                            total_tokens, rope_grid, sparsity, workspace, workspace_bytes, hip_stream);
}

}  // extern "C"

// ---- the block with MXFP4 linears ----

namespace {

struct BlockPlanMX4 {
    size_t mod, h, h4, hs, qkv, o, o4, os, x1, a, a4, as, attn, total;
};

BlockPlanMX4 block_plan_mx4(const h3_dit_dims* d, int32_t num_seqs, int32_t total_tokens) {
    BlockPlanMX4 p;
    const size_t n = static_cast<size_t>(total_tokens), c = static_cast<size_t>(d->hidden);
    const size_t f = static_cast<size_t>(d->ffn_dim);
    p.mod = align_up(static_cast<size_t>(num_seqs) * 6 * c * sizeof(float));
    p.h = align_up(n * c * 2);           // h, then h2 (bf16)
    p.h4 = align_up(n * c / 2);          // their MXFP4 codes
    p.hs = align_up(n * c / 32);
    p.qkv = align_up(n * 3 * c * 2);
    p.o = align_up(n * c * 2);
    p.o4 = align_up(n * c / 2);
    p.os = align_up(n * c / 32);
    p.x1 = align_up(n * c * 2);
    p.a = align_up(n * f * 2);
    p.a4 = align_up(n * f / 2);
    p.as = align_up(n * f / 32);
    p.attn = attn_plan(num_seqs, total_tokens, d->num_heads, d->head_dim, H3_ATTN_BF16).total;
    p.total = p.mod + p.h + p.h4 + p.hs + p.qkv + p.o + p.o4 + p.os + p.x1 + p.a + p.a4 + p.as + p.attn;
    return p;
}

h3_status check_dims_mx4(const h3_dit_dims* d, int32_t total_tokens) {
    h3_status st = check_dims(d);
    if (st != H3_OK) return st;
    if (d->ffn_dim % 256) return fail(H3_ERR_UNSUPPORTED, "ffn_dim=%d must be a multiple of 256 (MXFP4)", d->ffn_dim);
    const int64_t widest = std::max<int64_t>(3 * static_cast<int64_t>(d->hidden), d->ffn_dim);
    if (static_cast<int64_t>(total_tokens) * widest / 32 > INT32_MAX ||
        widest * std::max(d->hidden, d->ffn_dim) / 32 > INT32_MAX)
        return fail(H3_ERR_UNSUPPORTED, "MX scale arrays exceed 2^31 bytes");
    return ok();
}

}  // namespace

extern "C" {

H3_API size_t h3_dit_block_mx4_workspace_size(const h3_dit_dims* dims, int32_t num_seqs,
                                              int32_t total_tokens) {
    if (dims == nullptr || num_seqs < 0 || total_tokens < 0) return 0;
    if (check_dims_mx4(dims, total_tokens) != H3_OK) return 0;
    return block_plan_mx4(dims, num_seqs, total_tokens).total;
}

H3_API h3_status h3_dit_block_forward_mxfp4(const void* x, void* x_out, const void* cond,
                                            const h3_dit_mx_weights* weights,
                                            const h3_dit_dims* dims,
                                            const int32_t* cu_seqlens_dev,
                                            const int32_t* cu_seqlens_host, int32_t num_seqs,
                                            int32_t total_tokens, const int32_t* rope_grid,
                                            void* workspace, size_t workspace_bytes,
                                            void* hip_stream) {
    h3_status st = check_dims_mx4(dims, total_tokens);
    if (st != H3_OK) return st;
    st = check_cu(cu_seqlens_host, num_seqs, total_tokens);
    if (st != H3_OK) return st;
    if (total_tokens == 0) return ok();
    if (!x || !x_out || !cond || !weights || !cu_seqlens_dev || !rope_grid)
        return fail(H3_ERR_INVALID_ARGUMENT, "NULL pointer");
    const h3_dit_mx_weights& w = *weights;
    const h3_mx_matrix* mats[5] = {&w.w_qkv, &w.w_o, &w.w_gate, &w.w_up, &w.w_down};
    if (!w.w_mod || !w.q_norm || !w.k_norm) return fail(H3_ERR_INVALID_ARGUMENT, "NULL weight pointer");
    for (const h3_mx_matrix* m : mats) {
        if (!m->codes || !m->scales) return fail(H3_ERR_INVALID_ARGUMENT, "NULL MX weight pointer");
        if (!mx4_aligned(m->codes, m->scales))
            return fail(H3_ERR_UNSUPPORTED, "MXFP4 weight codes 16-byte and scales 8-byte aligned");
    }
    if (x == x_out) return fail(H3_ERR_INVALID_ARGUMENT, "x and x_out may not alias");
    const uintptr_t al = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(x_out) |
                         reinterpret_cast<uintptr_t>(cond) | reinterpret_cast<uintptr_t>(w.w_mod) |
                         reinterpret_cast<uintptr_t>(w.q_norm) | reinterpret_cast<uintptr_t>(w.k_norm);
    if (al & 15) return fail(H3_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
    const BlockPlanMX4 p = block_plan_mx4(dims, num_seqs, total_tokens);
    if (workspace_bytes < p.total || workspace == nullptr)
        return fail(H3_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, p.total);
    if (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))
        return fail(H3_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");

    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    char* ws = static_cast<char*>(workspace);
    auto carve = [&](size_t bytes) { char* r = ws; ws += bytes; return r; };
    float* mod = reinterpret_cast<float*>(carve(p.mod));
    uint16_t* hb = reinterpret_cast<uint16_t*>(carve(p.h));
    uint8_t* h4 = reinterpret_cast<uint8_t*>(carve(p.h4));
    uint8_t* hs = reinterpret_cast<uint8_t*>(carve(p.hs));
    uint16_t* qkv = reinterpret_cast<uint16_t*>(carve(p.qkv));
    uint16_t* obuf = reinterpret_cast<uint16_t*>(carve(p.o));
    uint8_t* o4 = reinterpret_cast<uint8_t*>(carve(p.o4));
    uint8_t* os = reinterpret_cast<uint8_t*>(carve(p.os));
    uint16_t* x1 = reinterpret_cast<uint16_t*>(carve(p.x1));
    uint16_t* ab = reinterpret_cast<uint16_t*>(carve(p.a));
    uint8_t* a4 = reinterpret_cast<uint8_t*>(carve(p.a4));
    uint8_t* as = reinterpret_cast<uint8_t*>(carve(p.as));
    void* attn_ws = carve(p.attn);

    const int64_t n = total_tokens, c = dims->hidden, ffn = dims->ffn_dim;
    const int64_t ms = 6 * c;
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    uint16_t* yb = static_cast<uint16_t*>(x_out);
    auto u8 = [](const void* ptr) { return static_cast<const uint8_t*>(ptr); };
    hipError_t e;
#define H3_TRY(call, what)                          \
    e = (call);                                     \
    if (e != hipSuccess) return hip_fail(e, what);

    H3_TRY(h3::launch_modulation(static_cast<const uint16_t*>(cond),
                                 static_cast<const uint16_t*>(w.w_mod), mod, num_seqs,
                                 static_cast<int>(c), stream), "modulation");
    H3_TRY(h3::launch_adaln(xb, hb, mod + 0 * c, mod + 1 * c, ms, cu_seqlens_dev, num_seqs, total_tokens,
                            static_cast<int>(c), dims->eps, stream), "adaln 1");
    H3_TRY(h3::launch_mx4_quantize(hb, c, n, c, h4, hs, stream), "h quantize");
    H3_TRY(h3::launch_gemm_mx4(h3::kEpiStore, h4, hs, u8(w.w_qkv.codes), u8(w.w_qkv.scales), nullptr,
                               nullptr, qkv, n, 3 * c, c, nullptr, nullptr, 0, nullptr, 1, stream),
           "qkv gemm");
    H3_TRY(h3::launch_qk_norm_rope(qkv, qkv + c, 3 * c, 3 * c,
                                   static_cast<const uint16_t*>(w.q_norm),
                                   static_cast<const uint16_t*>(w.k_norm), rope_grid,
                                   total_tokens, dims->num_heads, dims->head_dim,
                                   dims->rope_split, dims->rope_theta, dims->eps, stream),
           "qk norm rope");
    h3_status ast = run_attention(qkv, qkv + c, qkv + 2 * c, obuf, 3 * c, 3 * c, 3 * c, c,
                                  cu_seqlens_dev, cu_seqlens_host, num_seqs, total_tokens,
                                  dims->num_heads, dims->head_dim, nullptr, attn_ws, stream);
    if (ast != H3_OK) return ast;
    H3_TRY(h3::launch_mx4_quantize(obuf, c, n, c, o4, os, stream), "o quantize");
    H3_TRY(h3::launch_gemm_mx4(h3::kEpiGatedResidual, o4, os, u8(w.w_o.codes), u8(w.w_o.scales), nullptr,
                               nullptr, x1, n, c, c, xb, mod + 2 * c, ms, cu_seqlens_dev, num_seqs, stream),
           "out-proj gemm");
    H3_TRY(h3::launch_adaln(x1, hb, mod + 3 * c, mod + 4 * c, ms, cu_seqlens_dev, num_seqs, total_tokens,
                            static_cast<int>(c), dims->eps, stream), "adaln 2");
    H3_TRY(h3::launch_mx4_quantize(hb, c, n, c, h4, hs, stream), "h2 quantize");
    H3_TRY(h3::launch_gemm_mx4(h3::kEpiSwiGLU, h4, hs, u8(w.w_gate.codes), u8(w.w_gate.scales),
                               u8(w.w_up.codes), u8(w.w_up.scales), ab, n, ffn, c, nullptr, nullptr, 0,
                               nullptr, 1, stream), "gate/up gemm");
    H3_TRY(h3::launch_mx4_quantize(ab, ffn, n, ffn, a4, as, stream), "a quantize");
    H3_TRY(h3::launch_gemm_mx4(h3::kEpiGatedResidual, a4, as, u8(w.w_down.codes), u8(w.w_down.scales),
                               nullptr, nullptr, yb, n, c, ffn, x1, mod + 5 * c, ms, cu_seqlens_dev,
                               num_seqs, stream), "down gemm");
#undef H3_TRY
    return ok();
}

}  // extern "C"
