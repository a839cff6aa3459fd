// Prologue kernels of the QSA layer (HBM-bound elementwise work).
//
//  * kv_pool_kernel: for each micro-block touched by a chunk, rotate the
//    chunk's keys into the blocked K~ cache, transpose values into the blocked
//    V cache, and -- if the block becomes complete in this chunk -- mean-pool
//    its 4 raw indexer keys and rotate the mean at the block start (PyTorchKR
//    post "Qwen3.8-Flash-Next, 1/9의 학습 비용으로 …", section "QSA: 인덱서 자체의
//    비용을 줄이는 희소 어텐션": non-overlapping r-token micro-blocks, mean
//    pooling, compression before the positional encoding, one block-start
//    position per pooled key).
//  * kpend_store_kernel: keep the raw indexer keys of a trailing incomplete
//    block for the next call.
//  * qidx_rotate_kernel: rotate the indexer queries at their positions.
//  * token_keys_kernel: token-level indexer keys (r = 1), rotated at their
//    own positions, for the indexer QSA's pooled one is measured against.
//
// All rotations follow one fp32 recipe (each product and sum rounded, then
// bf16 round-to-nearest-even); the library is built with -ffp-contract=off.
#include "qsa_common.h"

namespace qsa {

// One wave per (sequence, touched block).
//   lanes 0..63 : head g = lane / 32, 8-dim chunk c = lane % 32 of K and V
//   lanes 0..15 : additionally 8-dim chunk of the pooled indexer key
__global__ __launch_bounds__(64) void kv_pool_kernel(
    Tables tab, int64_t L, int64_t q_offset, int64_t nblk_cap,
    const bf16_t *__restrict__ k, const bf16_t *__restrict__ v, const bf16_t *__restrict__ k_idx,
    bf16_t *__restrict__ k_cache, bf16_t *__restrict__ v_cache,
    bf16_t *__restrict__ kbar, const bf16_t *__restrict__ kpend, int do_kv, int do_pool)
{
    const int lane = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t blk = q_offset / kBlock + blockIdx.x;
    const int64_t t0 = blk * kBlock;                 // first token of the block
    const int64_t end = q_offset + L;

    if (do_kv) {
        const int g = lane >> 5;
        const int c = lane & 31;                     // dims 8c .. 8c+7
        const int partner = (c < 8) ? (c ^ 4) : c;   // rotary pairs: chunk c <-> c +/- 4
        const int64_t base = kcache_block_base(b, g, blk, nblk_cap);
        uint32_t vt[4][4];                           // [token][dim pair] for the V transpose
        bool have[4];
        for (int t = 0; t < kBlock; ++t) {
            const int64_t pos = t0 + t;
            have[t] = pos >= q_offset && pos < end;
            if (!have[t]) continue;
            const int64_t row = (b * L + (pos - q_offset)) * kKVHeads + g;
            u32x4 kx = *reinterpret_cast<const u32x4 *>(k + row * kHeadDim + 8 * c);
            u32x4 vx = *reinterpret_cast<const u32x4 *>(v + row * kHeadDim + 8 * c);
            if (c < 8) {
                u32x4 kp = *reinterpret_cast<const u32x4 *>(k + row * kHeadDim + 8 * partner);
                const float *cs = tab.cos + pos * kPairs;
                const float *sn = tab.sin + pos * kPairs;
                const bool first_half = c < 4;
                const int j0 = 8 * (c & 3);
                uint32_t outw[4];
                for (int i = 0; i < 4; ++i) {
                    float me_lo = __uint_as_float(kx[i] << 16), me_hi = __uint_as_float(kx[i] & 0xFFFF0000u);
                    float pa_lo = __uint_as_float(kp[i] << 16), pa_hi = __uint_as_float(kp[i] & 0xFFFF0000u);
                    float r[2];
                    for (int e = 0; e < 2; ++e) {
                        float me = e ? me_hi : me_lo, pa = e ? pa_hi : pa_lo;
                        float a = first_half ? me : pa;     // x_j
                        float bb = first_half ? pa : me;    // x_{j+32}
                        const int j = j0 + 2 * i + e;
                        rotate_pair(a, bb, cs[j], sn[j]);
                        r[e] = first_half ? a : bb;
                    }
                    outw[i] = pack_bf16x2(r[0], r[1]);
                }
                kx = u32x4{outw[0], outw[1], outw[2], outw[3]};
            }
            *reinterpret_cast<u32x4 *>(k_cache + base + kblock_off(t, 8 * c)) = kx;
            for (int i = 0; i < 4; ++i) vt[t][i] = vx[i];
        }
        // V block layout [d][t]: dims 8c..8c+7, 4 tokens each -> 64 contiguous bytes
        bf16_t *vb = v_cache + base + vblock_off(0, 8 * c);
        const bool full = have[0] && have[1] && have[2] && have[3];
        if (full) {
            u32x4 w0, w1, w2, w3;
            uint32_t o[16];
            for (int d = 0; d < 8; ++d) {
                const int i = d >> 1, sh = (d & 1) * 16;
                uint32_t e0 = (vt[0][i] >> sh) & 0xFFFFu, e1 = (vt[1][i] >> sh) & 0xFFFFu;
                uint32_t e2 = (vt[2][i] >> sh) & 0xFFFFu, e3 = (vt[3][i] >> sh) & 0xFFFFu;
                o[2 * d] = e0 | (e1 << 16);
                o[2 * d + 1] = e2 | (e3 << 16);
            }
            w0 = u32x4{o[0], o[1], o[2], o[3]};
            w1 = u32x4{o[4], o[5], o[6], o[7]};
            w2 = u32x4{o[8], o[9], o[10], o[11]};
            w3 = u32x4{o[12], o[13], o[14], o[15]};
            u32x4 *dst = reinterpret_cast<u32x4 *>(vb);
            dst[0] = w0; dst[1] = w1; dst[2] = w2; dst[3] = w3;
        } else {
            for (int t = 0; t < kBlock; ++t) {
                if (!have[t]) continue;
                for (int d = 0; d < 8; ++d)
                    vb[vblock_off(t, d)] = static_cast<bf16_t>((vt[t][d >> 1] >> ((d & 1) * 16)) & 0xFFFFu);
            }
        }
    }

    // Pooled indexer key of a block that is complete after this chunk.
    if (do_pool && lane < 16 && t0 + kBlock - 1 < end && t0 + kBlock - 1 >= q_offset) {
        const int c = lane;                          // dims 8c .. 8c+7 of 128
        const int partner = (c < 8) ? (c ^ 4) : c;
        float acc[8], accp[8];
        for (int t = 0; t < kBlock; ++t) {
            const int64_t pos = t0 + t;
            const bf16_t *src = (pos >= q_offset) ? k_idx + (b * L + (pos - q_offset)) * kIdxDim
                                                  : kpend + (b * kBlock + t) * kIdxDim;
            u32x4 x = *reinterpret_cast<const u32x4 *>(src + 8 * c);
            u32x4 xp = *reinterpret_cast<const u32x4 *>(src + 8 * partner);
            for (int i = 0; i < 4; ++i) {
                float lo = __uint_as_float(x[i] << 16), hi = __uint_as_float(x[i] & 0xFFFF0000u);
                float plo = __uint_as_float(xp[i] << 16), phi = __uint_as_float(xp[i] & 0xFFFF0000u);
                if (t == 0) {
                    acc[2 * i] = lo; acc[2 * i + 1] = hi; accp[2 * i] = plo; accp[2 * i + 1] = phi;
                } else {                             // token order, fp32 rounding at each step
                    acc[2 * i] += lo; acc[2 * i + 1] += hi; accp[2 * i] += plo; accp[2 * i + 1] += phi;
                }
            }
        }
        uint32_t outw[4];
        const int64_t pos = t0;                      // block-start position
        const float *cs = tab.cos + pos * kPairs;
        const float *sn = tab.sin + pos * kPairs;
        const bool first_half = c < 4;
        const int j0 = 8 * (c & 3);
        float r[8];
        for (int d = 0; d < 8; ++d) {
            float me = acc[d] * 0.25f;
            if (c < 8) {
                float pa = accp[d] * 0.25f;
                float a = first_half ? me : pa;
                float bb = first_half ? pa : me;
                rotate_pair(a, bb, cs[j0 + d], sn[j0 + d]);
                me = first_half ? a : bb;
            }
            r[d] = me;
        }
        for (int i = 0; i < 4; ++i) outw[i] = pack_bf16x2(r[2 * i], r[2 * i + 1]);
        *reinterpret_cast<u32x4 *>(kbar + (b * nblk_cap + blk) * kIdxDim + 8 * c) =
            u32x4{outw[0], outw[1], outw[2], outw[3]};
    }
}

// Raw indexer keys of the trailing incomplete block (positions 4*floor(end/4)
// .. end-1 that lie in the chunk) go to kpend[b][pos % 4].  One wave per sequence.
__global__ __launch_bounds__(64) void kpend_store_kernel(int64_t L, int64_t q_offset,
                                                         const bf16_t *__restrict__ k_idx,
                                                         bf16_t *__restrict__ kpend)
{
    const int64_t b = blockIdx.x;
    const int64_t end = q_offset + L;
    const int64_t start = (end / kBlock) * kBlock;
    const int lane = threadIdx.x;                    // 4 tokens x 16 chunks
    const int t = lane >> 4, c = lane & 15;
    const int64_t pos = start + t;
    if (pos >= end || pos < q_offset) return;
    *reinterpret_cast<u32x4 *>(kpend + (b * kBlock + t) * kIdxDim + 8 * c) =
        *reinterpret_cast<const u32x4 *>(k_idx + (b * L + (pos - q_offset)) * kIdxDim + 8 * c);
}

// Rotated indexer queries: qrot[b][i][h][128] = bf16(rotate(q_idx[b][i][h], pos_i)).
// pos_i = q_offset + i, or cache_len[b] when cache_len != nullptr (decode, L = 1).
// One thread per (token, head, 8-dim chunk).
__global__ __launch_bounds__(256) void qidx_rotate_kernel(Tables tab, int32_t B, int64_t L, int64_t q_offset,
                                                          const int32_t *__restrict__ cache_len,
                                                          const bf16_t *__restrict__ q_idx,
                                                          bf16_t *__restrict__ qrot)
{
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = static_cast<int64_t>(B) * L * kIdxHeads * 16;
    if (gid >= total) return;
    const int c = static_cast<int>(gid & 15);
    const int64_t row = gid >> 4;                    // (b, i, h)
    const int64_t bi = row / kIdxHeads;              // (b, i)
    const int64_t b = bi / L;
    const int64_t pos = cache_len ? static_cast<int64_t>(cache_len[b]) : q_offset + (bi - b * L);
    const bf16_t *src = q_idx + row * kIdxDim;
    u32x4 x = *reinterpret_cast<const u32x4 *>(src + 8 * c);
    if (c < 8) {
        const int partner = c ^ 4;
        u32x4 xp = *reinterpret_cast<const u32x4 *>(src + 8 * partner);
        const float *cs = tab.cos + pos * kPairs;
        const float *sn = tab.sin + pos * kPairs;
        const bool first_half = c < 4;
        const int j0 = 8 * (c & 3);
        uint32_t outw[4];
        for (int i = 0; i < 4; ++i) {
            float r[2];
            for (int e = 0; e < 2; ++e) {
                float me = __uint_as_float(e ? (x[i] & 0xFFFF0000u) : (x[i] << 16));
                float pa = __uint_as_float(e ? (xp[i] & 0xFFFF0000u) : (xp[i] << 16));
                float a = first_half ? me : pa;
                float bb = first_half ? pa : me;
                rotate_pair(a, bb, cs[j0 + 2 * i + e], sn[j0 + 2 * i + e]);
                r[e] = first_half ? a : bb;
            }
            outw[i] = pack_bf16x2(r[0], r[1]);
        }
        x = u32x4{outw[0], outw[1], outw[2], outw[3]};
    }
    *reinterpret_cast<u32x4 *>(qrot + row * kIdxDim + 8 * c) = x;
}

// Token-level indexer keys (r = 1): the indexer key of position q_offset + i,
// rotated at that position, goes to ktok[b][q_offset + i] (no pooling).
// 16 threads per token, 8 dims each.
__global__ __launch_bounds__(256) void token_keys_kernel(Tables tab, int32_t B, int64_t L, int64_t q_offset,
                                                         int64_t tok_cap, const bf16_t *__restrict__ k_idx,
                                                         bf16_t *__restrict__ ktok)
{
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = static_cast<int64_t>(B) * L * 16;
    if (gid >= total) return;
    const int c = static_cast<int>(gid & 15);
    const int64_t row = gid >> 4;                    // (b, i)
    const int64_t b = row / L;
    const int64_t pos = q_offset + (row - b * L);
    const bf16_t *src = k_idx + row * kIdxDim;
    u32x4 x = *reinterpret_cast<const u32x4 *>(src + 8 * c);
    if (c < 8) {
        const u32x4 xp = *reinterpret_cast<const u32x4 *>(src + 8 * (c ^ 4));
        const float *cs = tab.cos + pos * kPairs;
        const float *sn = tab.sin + pos * kPairs;
        const bool first_half = c < 4;
        const int j0 = 8 * (c & 3);
        uint32_t outw[4];
        for (int i = 0; i < 4; ++i) {
            float r[2];
            for (int e = 0; e < 2; ++e) {
                float me = __uint_as_float(e ? (x[i] & 0xFFFF0000u) : (x[i] << 16));
                float pa = __uint_as_float(e ? (xp[i] & 0xFFFF0000u) : (xp[i] << 16));
                float a = first_half ? me : pa;
                float bb = first_half ? pa : me;
                rotate_pair(a, bb, cs[j0 + 2 * i + e], sn[j0 + 2 * i + e]);
                r[e] = first_half ? a : bb;
            }
            outw[i] = pack_bf16x2(r[0], r[1]);
        }
        x = u32x4{outw[0], outw[1], outw[2], outw[3]};
    }
    *reinterpret_cast<u32x4 *>(ktok + (b * tok_cap + pos) * kIdxDim + 8 * c) = x;
}

// ---------------------------------------------------------------- launchers
hipError_t launch_kv_pool(const Tables &tab, hipStream_t st, int32_t B, int64_t L, int64_t q_offset,
                          int64_t nblk_cap, const bf16_t *k, const bf16_t *v, const bf16_t *k_idx,
                          bf16_t *k_cache, bf16_t *v_cache, bf16_t *kbar, const bf16_t *kpend,
                          bool do_kv, bool do_pool)
{
    if (L <= 0) return hipSuccess;
    const int64_t first = q_offset / kBlock;
    const int64_t last = (q_offset + L - 1) / kBlock;
    const int64_t nblocks = last - first + 1;
    dim3 grid(static_cast<unsigned>(nblocks), static_cast<unsigned>(B));
    hipLaunchKernelGGL(kv_pool_kernel, grid, dim3(64), 0, st, tab, L, q_offset, nblk_cap, k, v, k_idx,
                       k_cache, v_cache, kbar, kpend, do_kv ? 1 : 0, do_pool ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_kpend_store(hipStream_t st, int32_t B, int64_t L, int64_t q_offset, const bf16_t *k_idx,
                              bf16_t *kpend)
{
    if (L <= 0 || (q_offset + L) % kBlock == 0) return hipSuccess;
    hipLaunchKernelGGL(kpend_store_kernel, dim3(B), dim3(64), 0, st, L, q_offset, k_idx, kpend);
    return hipGetLastError();
}

hipError_t launch_qidx_rotate(const Tables &tab, hipStream_t st, int32_t B, int64_t L, int64_t q_offset,
                              const int32_t *cache_len, const bf16_t *q_idx, bf16_t *qrot)
{
    const int64_t total = static_cast<int64_t>(B) * L * kIdxHeads * 16;
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(qidx_rotate_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, tab, B, L,
                       q_offset, cache_len, q_idx, qrot);
    return hipGetLastError();
}

hipError_t launch_token_keys(const Tables &tab, hipStream_t st, int32_t B, int64_t L, int64_t q_offset, int64_t tok_cap,
                             const bf16_t *k_idx, bf16_t *ktok)
{
    const int64_t total = static_cast<int64_t>(B) * L * 16;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(token_keys_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, st, tab, B, L,
                       q_offset, tok_cap, k_idx, ktok);
    return hipGetLastError();
}

}  // namespace qsa
