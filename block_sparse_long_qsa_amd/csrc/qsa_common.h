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
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Decode score scan geometry: each wave streams bpw consecutive keys (a
// multiple of 64, at most kScanBlocksPerWaveMax, chosen per call), a
// work-group of 4 waves 4*bpw; each work-group leaves a summary of its score
// histogram in a slot of 1 + kSumWords words (see decode_scan_kernel).
constexpr int kScanBlocksPerWaveMax = 2048;
constexpr int kSumWords = kMaxBudget;
constexpr int kSumSlot = 1 + kSumWords;

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


// ---- wave-level helpers (64-lane wavefronts)

// Order this wave's LDS accesses: a write by one lane is seen by a later read of
// another lane.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Number of set lanes of m below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// Value of lane (lane ^ X) of this wave.  X < 16 moves data inside the
// VALU with DPP: quad permutations for 1 and 2; 4 = half-row mirror then quad
// reversal; 8 = row mirror then half-row mirror.  Larger X use ds_bpermute.
template <int X>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
    const int x = static_cast<int>(v);
    if constexpr (X == 1) {
        return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
    } else if constexpr (X == 2) {
        return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
    } else if constexpr (X == 4) {
        const int t = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);                 // half mirror
        return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, t, 0x1B, 0xF, 0xF, false));  // [3,2,1,0]
    } else if constexpr (X == 8) {
        const int t = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);                 // row mirror
        return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, t, 0x141, 0xF, 0xF, false)); // half mirror
    } else {
        return static_cast<uint32_t>(__shfl_xor(x, X));
    }
}

// One bitonic merge step of (SIZE, STRIDE) and the smaller strides after it,
// over 64*R keys held lane-major: element lane*R + r sits in k[r] of that
// lane.  Strides below R compare registers of one lane; larger ones compare
// register r of lanes lane and lane ^ (STRIDE/R).
template <int R, int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_steps(uint32_t (&k)[R], int lane) {
    if constexpr (STRIDE < R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if ((r & STRIDE) == 0) {
                const bool desc = ((lane * R + r) & SIZE) == 0;
                const uint32_t x = k[r], y = k[r | STRIDE];
                const uint32_t hi = x > y ? x : y, lo = x > y ? y : x;
                k[r] = desc ? hi : lo;
                k[r | STRIDE] = desc ? lo : hi;
            }
        }
    } else {
        constexpr int X = STRIDE / R;
        const bool desc = ((lane * R) & SIZE) == 0;
        const bool lower = (lane & X) == 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t y = lane_xor<X>(k[r]);
            const uint32_t hi = k[r] > y ? k[r] : y, lo = k[r] > y ? y : k[r];
            k[r] = (lower == desc) ? hi : lo;
        }
    }
    if constexpr (STRIDE > 1) bitonic_steps<R, SIZE, STRIDE / 2>(k, lane);
}

template <int R, int SIZE>
__device__ __forceinline__ void bitonic_stages(uint32_t (&k)[R], int lane) {
    bitonic_steps<R, SIZE, SIZE / 2>(k, lane);
    if constexpr (SIZE < 64 * R) bitonic_stages<R, SIZE * 2>(k, lane);
}

// Bitonic sort of 64*R 32-bit keys held by one wave, descending: afterwards
// element lane*R + r (k[r] of lane `lane`) is the (lane*R + r)-th largest.
template <int R>
__device__ __forceinline__ void wave_sort_desc(uint32_t (&k)[R], int lane) {
    bitonic_stages<R, 2>(k, lane);
}

// Exclusive prefix sum of v over the NT threads of a workgroup (every thread
// calls it); total receives the sum over all threads.
template <int NT>
__device__ __forceinline__ uint32_t block_scan_nt(uint32_t v, uint32_t *wsum /* LDS [NT/64] */, uint32_t &total)
{
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = v;
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
    total = 0;
    for (int w = 0; w < NW; ++w) {
        if (w < wave) before += wsum[w];
        total += wsum[w];
    }
    __syncthreads();
    return before + incl - v;
}

// Write the n (<= 64*R) selected block ids of sel[] to out[] ascending.
template <int R>
__device__ __forceinline__ void emit_sorted(const int32_t *sel, int n, int32_t *__restrict__ out, int lane) {
    uint32_t k[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = r * 64 + lane;
        k[r] = (i < n) ? static_cast<uint32_t>(sel[i]) + 1u : 0u;     // ids + 1 sort ahead of the padding
    }
    wave_sort_desc<R>(k, lane);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = lane * R + r;
        if (i < n) out[n - 1 - i] = static_cast<int32_t>(k[r] - 1u);
    }
}

}  // namespace qsa
