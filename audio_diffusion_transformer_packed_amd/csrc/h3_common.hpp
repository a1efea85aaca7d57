// Shared device helpers for the gfx950 kernels of the packed DiT hot path.
// CDNA4: 64-lane wavefronts, bf16 MFMA 32x32x16 with fp32 accumulation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Native vectors for raw 16- and 8-byte moves (HIP's uint4 is a struct with a
// union inside, which can keep arrays of it out of registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// 16 bytes viewed as 8 bf16 / 4 words.
union Chunk16 {
    uint4 u;
    bf16x8 b;
    uint16_t h[8];
    uint32_t w[4];
};

union Chunk8 {
    uint2 u;
    bf16x4 b;
    uint16_t h[4];
    uint32_t w[2];
};

// Streaming (nontemporal) 16-byte global access for data touched once.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
__device__ __forceinline__ void store_stream16(void* p, uint4 v) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ float bf2f(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int off = width / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Work list index of workgroup b. Workgroup ids are dealt round-robin over
// the 8 XCDs (b runs on XCD b % 8), each with its own L2. With a list in
// (segment, head, query tile) order, consecutive ids would put the items of
// one head on all eight XCDs at once, and each XCD's L2 would fetch that
// head's K and V. When num_heads % 8 == 0 (and rank_prefix, the schedule's
// per-segment tile prefix in list order, is given) XCD x instead takes the
// items of heads x, x + 8, ... in list order, its (b / 8)-th such item being
// workgroup b's: the workgroups an XCD runs at one time then stream one
// head's K and V through its L2 together, and every segment's work still
// splits evenly over the XCDs. Otherwise the list order is kept. (Used by
// the dense attention kernels.)
__device__ __forceinline__ int64_t xcd_item(unsigned b, const int32_t* __restrict__ rank_prefix,
                                            int num_seqs, int num_heads) {
    if (rank_prefix == nullptr || (num_heads & 7) != 0) return b;
    const int x = static_cast<int>(b & 7);
    const int64_t kk = b >> 3;
    const int hpx = num_heads >> 3;
    // segment rank r: the largest with rank_prefix[r] * hpx <= kk
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (static_cast<int64_t>(__builtin_amdgcn_readfirstlane(rank_prefix[mid])) * hpx <= kk) lo = mid;
        else hi = mid - 1;
    }
    const int p0 = __builtin_amdgcn_readfirstlane(rank_prefix[lo]);
    const int tiles = __builtin_amdgcn_readfirstlane(rank_prefix[lo + 1]) - p0;
    // j < 2^29 (b is a 32-bit workgroup id): 32-bit division
    const unsigned j = static_cast<unsigned>(kk - static_cast<int64_t>(p0) * hpx);
    const unsigned hq = j / static_cast<unsigned>(tiles);
    const int64_t h = 8 * static_cast<int64_t>(hq) + x;
    return static_cast<int64_t>(p0) * num_heads + h * tiles + (j - hq * static_cast<unsigned>(tiles));
}

// Segment of token t: largest s with cu[s] <= t (cu non-decreasing, cu[0] = 0).
__device__ __forceinline__ int find_segment(const int32_t* __restrict__ cu, int num_seqs,
                                            int64_t t) {
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (static_cast<int64_t>(cu[mid]) <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}


// ---- MXFP8 (OCP MX v1.0: 32-element blocks, E8M0 scale, E4M3 elements) ----
// E8M0 byte of a block's scale 2^(floor(log2 amax) - 8) from its fp32 amax,
// never below 2^-127: the exponent field minus 8, clamped at 0 (zero and
// fp32-subnormal amax give byte 0).
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
    const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xff);
    return static_cast<uint32_t>(max(e - 8, 0));
}
// 1 / scale for that byte, 2^(127 - byte), built from its bits.
__device__ __forceinline__ float mx_inv_scale(uint32_t byte) {
    return __uint_as_float((254u - byte) << 23);
}
// E4M3 codes (byte i = value i) of eight values already divided by the
// scale: saturated to +-448, then round to nearest even.
__device__ __forceinline__ uint2 mx_codes8(const float (&v)[8]) {
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = fminf(fmaxf(v[i], -448.0f), 448.0f);
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], w1, true);
    return make_uint2(static_cast<uint32_t>(w0), static_cast<uint32_t>(w1));
}
// Byte offset of the scale of row r, block j in the K-step-major layout
// (the four scales of a row for one 128-element K step form one dword).
__device__ __forceinline__ int64_t mx_scale_offset(int64_t r, int64_t j, int64_t rows) {
    return ((j >> 2) * rows + r) * 4 + (j & 3);
}

// ---- MXFP4 (OCP MX v1.0: 32-element blocks, E8M0 scale, E2M1 elements) ----
// E8M0 byte of a block's scale 2^(floor(log2 amax) - 2) from its fp32 amax:
// the exponent field minus 2, clamped at 0.
__device__ __forceinline__ uint32_t mx4_scale_byte(float amax) {
    const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xff);
    return static_cast<uint32_t>(max(e - 2, 0));
}
// 4-bit E2M1 codes of eight values already divided by the scale (|v| < 8),
// element 2i in the low nibble of byte i. A code is the index of the nearest
// of 0, 0.5, 1, 1.5, 2, 3, 4, 6 (midpoints to the even index, saturating at
// 6) plus 8 when v is negative (zero included). v_cvt_scalef32_pk_fp4_f32 at
// scale 1 rounds exactly so: checked on gfx950 against that rule for every
// bf16 value below 8 in magnitude, the inputs this sees (bf16 times a power
// of two).
__device__ __forceinline__ uint32_t e2m1x8(const float (&v)[8]) {
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
}
// Byte offset of the scale of row r, block j in the MXFP4 K-step-major
// layout: 8 bytes per row and 256-element K step, the step's even blocks
// (0, 2, 4, 6) in its first dword and the odd ones in the second.
__device__ __forceinline__ int64_t mx4_scale_offset(int64_t r, int64_t j, int64_t rows) {
    return ((j >> 3) * rows + r) * 8 + (j & 1) * 4 + ((j & 7) >> 1);
}

}  // namespace h3
