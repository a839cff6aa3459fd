// Shared definitions of the gfx950 QSA kernels and the host library.
// Shapes are those of the QSA layer on the PyTorchKR post "Qwen3.8-Flash-Next,
// 1/9의 학습 비용으로 Qwen3.7-Plus(397B-A17B) 수준에 도달한 125B-A6B 모델" (spec
// table rows "Qwen Sparse Attention", "QSA 인덱서", "QSA 예산").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

constexpr int kQHeads = 24;       // core query heads
constexpr int kKVHeads = 2;       // core KV heads
constexpr int kGroup = 12;        // query heads per KV head
constexpr int kHeadDim = 256;
constexpr int kRopeDim = 64;      // rotated dims of a core head
constexpr int kPairs = 32;        // rotary frequency pairs (j, j + 32)
constexpr int kIdxHeads = 4;
constexpr int kIdxDim = 128;
constexpr int kBlock = 4;         // micro-block size r
constexpr int kMaxBudget = 512;   // blocks

// One micro-block of one head in the K~ / V caches: 4 tokens x 256 dims bf16.
constexpr int kBlockElems = kBlock * kHeadDim;   // 1024 bf16 = 2 KiB

typedef uint16_t bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Handle contents visible to the launchers.
struct Tables {
    const float *cos;   // [max_ctx][32]
    const float *sin;   // [max_ctx][32]
};

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Rotate one rotary pair (a, b) = (x_j, x_{j+32}) by the angle with cosine c
// and sine s.  The library is compiled with -ffp-contract=off, so each product
// and sum below is a separately rounded fp32 operation.
__device__ __forceinline__ void rotate_pair(float &a, float &b, float c, float s) {
    float ac = a * c;
    float bs = b * s;
    float bc = b * c;
    float as = a * s;
    a = ac - bs;
    b = bc + as;
}

// Decode position of sequence b: cache_len[b] clamped to [0, bound] so that a
// bad length can never address memory outside the caches or tables.
__device__ __forceinline__ int64_t decode_pos(const int32_t *cache_len, int64_t b, int64_t bound) {
    int64_t p = cache_len[b];
    return p < 0 ? 0 : (p > bound ? bound : p);
}

// Offsets inside the blocked caches (elements).
__device__ __forceinline__ int64_t kcache_block_base(int64_t b, int g, int64_t blk, int64_t nblk_cap) {
    return ((b * kKVHeads + g) * nblk_cap + blk) * kBlockElems;
}
// element (token t in block, dim d) of a K~ block: [d/32][t][d%32]
__device__ __forceinline__ int kblock_off(int t, int d) { return ((d >> 5) * kBlock + t) * 32 + (d & 31); }
// element (token t in block, dim d) of a V block: [d][t]
__device__ __forceinline__ int vblock_off(int t, int d) { return d * kBlock + t; }

}  // namespace qsa
