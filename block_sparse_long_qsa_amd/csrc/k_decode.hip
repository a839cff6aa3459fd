// Decode kernels: append one token per sequence and scan the pooled indexer
// keys (PyTorchKR post "Qwen3.8-Flash-Next, 1/9의 학습 비용으로 …", section "QSA:
// 인덱서 자체의 비용을 줄이는 희소 어텐션": the indexer compares the query with the
// mean-pooled, block-start-rotated keys of fully observed blocks, so one
// decode step reads n/4 pooled keys instead of n token keys).
#include "qsa_common.h"

namespace qsa {

constexpr int kDecodeBins = 2048;      // histogram of score bits 30..20 per sequence

// One wave per sequence.  p = cache_len[b]:
//   lanes: head g = lane/32, chunk c = lane%32 -> rotate k at p into K~ slot p%4
//          and copy v into V slot p%4 (when k is given);
//   lanes 0..15: raw k_idx into kpend[p%4]; when p%4 == 3 pool the completed
//          block (kpend slots 0..2 + this token) into kbar;
//   lanes: head lane/16, chunk lane%16 -> rotated q_idx at p into qrot (when
//          q_idx is given).
__global__ __launch_bounds__(64) void decode_append_kernel(
    Tables tab, const int32_t *__restrict__ cache_len, int64_t ctx_bound, int64_t nblk_cap,
    const bf16_t *__restrict__ k, const bf16_t *__restrict__ v, const bf16_t *__restrict__ k_idx,
    const bf16_t *__restrict__ q_idx,
    bf16_t *__restrict__ k_cache, bf16_t *__restrict__ v_cache, bf16_t *__restrict__ kbar,
    bf16_t *__restrict__ kpend, bf16_t *__restrict__ qrot, uint32_t *__restrict__ dhist)
{
    const int lane = threadIdx.x;
    const int64_t b = blockIdx.x;
    for (int x = lane; x < kDecodeBins; x += 64) dhist[b * kDecodeBins + x] = 0;   // filled by the scan
    const int64_t p = decode_pos(cache_len, b, ctx_bound);
    const int64_t blk = p / kBlock;
    const int t = static_cast<int>(p - blk * kBlock);
    const float *cs = tab.cos + p * kPairs;
    const float *sn = tab.sin + p * kPairs;

    if (k) {   // K~ and V (not needed when only the selection is wanted)
        const int g = lane >> 5, c = lane & 31;
        const int64_t row = b * kKVHeads + g;
        u32x4 kx = *reinterpret_cast<const u32x4 *>(k + row * kHeadDim + 8 * c);
        const u32x4 vx = *reinterpret_cast<const u32x4 *>(v + row * kHeadDim + 8 * c);
        if (c < 8) {
            const u32x4 kp = *reinterpret_cast<const u32x4 *>(k + row * kHeadDim + 8 * (c ^ 4));
            const bool first_half = c < 4;
            const int j0 = 8 * (c & 3);
            uint32_t w[4];
            for (int i = 0; i < 4; ++i) {
                float r[2];
                for (int e = 0; e < 2; ++e) {
                    float me = __uint_as_float(e ? (kx[i] & 0xFFFF0000u) : (kx[i] << 16));
                    float pa = __uint_as_float(e ? (kp[i] & 0xFFFF0000u) : (kp[i] << 16));
                    float a = first_half ? me : pa, bb = first_half ? pa : me;
                    rotate_pair(a, bb, cs[j0 + 2 * i + e], sn[j0 + 2 * i + e]);
                    r[e] = first_half ? a : bb;
                }
                w[i] = pack_bf16x2(r[0], r[1]);
            }
            kx = u32x4{w[0], w[1], w[2], w[3]};
        }
        const int64_t base = kcache_block_base(b, g, blk, nblk_cap);
        *reinterpret_cast<u32x4 *>(k_cache + base + kblock_off(t, 8 * c)) = kx;
        bf16_t *vb = v_cache + base;
        for (int d = 0; d < 8; ++d)
            vb[vblock_off(t, 8 * c + d)] = static_cast<bf16_t>((vx[d >> 1] >> ((d & 1) * 16)) & 0xFFFFu);
    }
    if (lane < 16) {   // indexer key: pending slot, and pooling of a completed block
        const int c = lane;
        const u32x4 x = *reinterpret_cast<const u32x4 *>(k_idx + b * kIdxDim + 8 * c);
        *reinterpret_cast<u32x4 *>(kpend + (b * kBlock + t) * kIdxDim + 8 * c) = x;
        if (t == kBlock - 1) {
            const int partner = (c < 8) ? (c ^ 4) : c;
            const u32x4 xp = *reinterpret_cast<const u32x4 *>(k_idx + b * kIdxDim + 8 * partner);
            float acc[8], accp[8];
            for (int s = 0; s < kBlock; ++s) {
                u32x4 y, yp;
                if (s < t) {
                    y = *reinterpret_cast<const u32x4 *>(kpend + (b * kBlock + s) * kIdxDim + 8 * c);
                    yp = *reinterpret_cast<const u32x4 *>(kpend + (b * kBlock + s) * kIdxDim + 8 * partner);
                } else {
                    y = x;
                    yp = xp;
                }
                for (int i = 0; i < 4; ++i) {
                    float lo = __uint_as_float(y[i] << 16), hi = __uint_as_float(y[i] & 0xFFFF0000u);
                    float plo = __uint_as_float(yp[i] << 16), phi = __uint_as_float(yp[i] & 0xFFFF0000u);
                    if (s == 0) {
                        acc[2 * i] = lo; acc[2 * i + 1] = hi; accp[2 * i] = plo; accp[2 * i + 1] = phi;
                    } else {
                        acc[2 * i] += lo; acc[2 * i + 1] += hi; accp[2 * i] += plo; accp[2 * i + 1] += phi;
                    }
                }
            }
            const float *bcs = tab.cos + (blk * kBlock) * kPairs;
            const float *bsn = tab.sin + (blk * kBlock) * kPairs;
            const bool first_half = c < 4;
            const int j0 = 8 * (c & 3);
            float r[8];
            for (int d = 0; d < 8; ++d) {
                float me = acc[d] * 0.25f;
                if (c < 8) {
                    float pa = accp[d] * 0.25f;
                    float a = first_half ? me : pa, bb = first_half ? pa : me;
                    rotate_pair(a, bb, bcs[j0 + d], bsn[j0 + d]);
                    me = first_half ? a : bb;
                }
                r[d] = me;
            }
            *reinterpret_cast<u32x4 *>(kbar + (b * nblk_cap + blk) * kIdxDim + 8 * c) =
                u32x4{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]),
                      pack_bf16x2(r[6], r[7])};
        }
    }
    if (q_idx) {   // rotated indexer query (not needed when a selection is reused)
        const int h = lane >> 4, c = lane & 15;
        const bf16_t *src = q_idx + (b * kIdxHeads + h) * kIdxDim;
        u32x4 x = *reinterpret_cast<const u32x4 *>(src + 8 * c);
        if (c < 8) {
            const u32x4 xp = *reinterpret_cast<const u32x4 *>(src + 8 * (c ^ 4));
            const bool first_half = c < 4;
            const int j0 = 8 * (c & 3);
            uint32_t w[4];
            for (int i = 0; i < 4; ++i) {
                float r[2];
                for (int e = 0; e < 2; ++e) {
                    float me = __uint_as_float(e ? (x[i] & 0xFFFF0000u) : (x[i] << 16));
                    float pa = __uint_as_float(e ? (xp[i] & 0xFFFF0000u) : (xp[i] << 16));
                    float a = first_half ? me : pa, bb = first_half ? pa : me;
                    rotate_pair(a, bb, cs[j0 + 2 * i + e], sn[j0 + 2 * i + e]);
                    r[e] = first_half ? a : bb;
                }
                w[i] = pack_bf16x2(r[0], r[1]);
            }
            x = u32x4{w[0], w[1], w[2], w[3]};
        }
        *reinterpret_cast<u32x4 *>(qrot + (b * kIdxHeads + h) * kIdxDim + 8 * c) = x;
    }
}

// 8 dims (chunk c of 16) of a 128-dim row rotated at one position: chunks
// 0..7 hold the rotary dims, chunk c pairs with c ^ 4 (dims j and j + 32).
__device__ __forceinline__ u32x4 rotate_chunk8(u32x4 x, u32x4 xp, int c, const float *cs, const float *sn) {
    if (c >= 8) return x;
    const bool first_half = c < 4;
    const int j0 = 8 * (c & 3);
    uint32_t w[4];
    for (int i = 0; i < 4; ++i) {
        float r[2];
        for (int e = 0; e < 2; ++e) {
            float me = __uint_as_float(e ? (x[i] & 0xFFFF0000u) : (x[i] << 16));
            float pa = __uint_as_float(e ? (xp[i] & 0xFFFF0000u) : (xp[i] << 16));
            float a = first_half ? me : pa, bb = first_half ? pa : me;
            rotate_pair(a, bb, cs[j0 + 2 * i + e], sn[j0 + 2 * i + e]);
            r[e] = first_half ? a : bb;
        }
        w[i] = pack_bf16x2(r[0], r[1]);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

// Token-level indexer step (r = 1), one wave per sequence, p = cache_len[b]:
// the new token's indexer key rotated at p goes to ktok[b][p], the indexer
// query rotated at p to qrot, and the sequence's score histogram is cleared.
__global__ __launch_bounds__(64) void token_decode_append_kernel(
    Tables tab, const int32_t *__restrict__ cache_len, int64_t ctx_bound, int64_t tok_cap,
    const bf16_t *__restrict__ k_idx, const bf16_t *__restrict__ q_idx, bf16_t *__restrict__ ktok,
    bf16_t *__restrict__ qrot, uint32_t *__restrict__ dhist)
{
    const int lane = threadIdx.x;
    const int64_t b = blockIdx.x;
    for (int x = lane; x < kDecodeBins; x += 64) dhist[b * kDecodeBins + x] = 0;
    const int64_t p = decode_pos(cache_len, b, ctx_bound);
    const float *cs = tab.cos + p * kPairs;
    const float *sn = tab.sin + p * kPairs;
    const int c = lane & 15, h = lane >> 4;
    {   // lanes 0..15: the key; the query's 4 heads over all 64 lanes
        const bf16_t *src = q_idx + (b * kIdxHeads + h) * kIdxDim;
        const u32x4 x = *reinterpret_cast<const u32x4 *>(src + 8 * c);
        const u32x4 xp = *reinterpret_cast<const u32x4 *>(src + 8 * (c ^ 4));
        *reinterpret_cast<u32x4 *>(qrot + (b * kIdxHeads + h) * kIdxDim + 8 * c) = rotate_chunk8(x, xp, c, cs, sn);
    }
    if (lane < 16) {
        const bf16_t *src = k_idx + b * kIdxDim;
        const u32x4 x = *reinterpret_cast<const u32x4 *>(src + 8 * c);
        const u32x4 xp = *reinterpret_cast<const u32x4 *>(src + 8 * (c ^ 4));
        *reinterpret_cast<u32x4 *>(ktok + (b * tok_cap + p) * kIdxDim + 8 * c) = rotate_chunk8(x, xp, c, cs, sn);
    }
}

// Score scan: scores[b][blk] = sum_h ReLU(<q~_h, k̄_blk>) for blk < floor(p/r),
// r = 1 << rsh (4: pooled micro-blocks; 1: one rotated key per token).
// v_mfma_f32_16x16x32_bf16 with A = q~ (4 real rows of 16), B = 16 pooled keys;
// lanes 0..15 end with the 4 heads of one block.  Each wave streams 512 blocks
// and collects their scores in LDS, then writes them with one 16-byte store per
// lane and 256 scores: 4-byte stores interleaved with the k̄ loads cost about 6%
// of the scan.
constexpr int kScanBlocksPerWave = 512;
constexpr int kScanBlocksPerWG = 4 * kScanBlocksPerWave;

// Each workgroup also histograms the top 11 value bits of its scores and adds
// the histogram to the sequence's (zeroed by decode_append_kernel).
__global__ __launch_bounds__(256) void decode_scan_kernel(const int32_t *__restrict__ cache_len, int64_t ctx_bound,
                                                          int rsh, int64_t nblk_cap,
                                                          int64_t ncol, const bf16_t *__restrict__ qrot,
                                                          const bf16_t *__restrict__ kbar,
                                                          float *__restrict__ scores, uint32_t *__restrict__ dhist)
{
    __shared__ uint32_t lh[kDecodeBins];
    __shared__ __attribute__((aligned(16))) uint32_t sl[4][kScanBlocksPerWave];   // each wave's score bits
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t b = blockIdx.y;
    const int64_t o = decode_pos(cache_len, b, ctx_bound) >> rsh;
    if (static_cast<int64_t>(blockIdx.x) * kScanBlocksPerWG >= o) return;     // whole workgroup idle
    for (int x = threadIdx.x; x < kDecodeBins; x += 256) lh[x] = 0;
    __syncthreads();
    const int64_t w0 = static_cast<int64_t>(blockIdx.x) * kScanBlocksPerWG + wave * kScanBlocksPerWave;
    if (w0 < o) {
    const int r = lane & 15, g = lane >> 4;
    bf16x8 af[4];
    for (int s = 0; s < 4; ++s) {
        if (r < kIdxHeads)
            af[s] = *reinterpret_cast<const bf16x8 *>(qrot + (b * kIdxHeads + r) * kIdxDim + 32 * s + 8 * g);
        else
            af[s] = bf16x8{};
    }
    const bf16_t *kb = kbar + b * nblk_cap * kIdxDim;
    const int64_t wend = (w0 + kScanBlocksPerWave < o) ? w0 + kScanBlocksPerWave : o;
    for (int64_t c0 = w0; c0 < wend; c0 += 64) {
        bf16x8 bf[4][4];
        for (int u = 0; u < 4; ++u) {
            int64_t blk = c0 + 16 * u + r;
            if (blk >= o) blk = w0;                      // in bounds; result discarded
            for (int s = 0; s < 4; ++s)
                bf[u][s] = *reinterpret_cast<const bf16x8 *>(kb + blk * kIdxDim + 32 * s + 8 * g);
        }
        for (int u = 0; u < 4; ++u) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], bf[u][s], acc, 0, 0, 0);
            const int64_t blk = c0 + 16 * u + r;
            if (g == 0 && blk < o) {
                float sc = fmaxf(acc[0], 0.f) + fmaxf(acc[1], 0.f) + fmaxf(acc[2], 0.f) + fmaxf(acc[3], 0.f);
                const uint32_t bits = __float_as_uint(sc) & 0x7FFFFFFFu;
                sl[wave][blk - w0] = bits;
                atomicAdd(&lh[bits >> 20], 1u);
            }
        }
    }
    }
    __syncthreads();
    if (w0 < o) {   // the wave's scores, blocks w0 .. wend-1
        const int64_t n = ((w0 + kScanBlocksPerWave < o) ? w0 + kScanBlocksPerWave : o) - w0;
        float *dst = scores + b * ncol + w0;
        const bool vec = ((b * ncol + w0) & 3) == 0;
        for (int i = 4 * lane; i < n; i += 256) {
            if (vec && i + 3 < n)
                *reinterpret_cast<u32x4 *>(dst + i) = *reinterpret_cast<const u32x4 *>(&sl[wave][i]);
            else
                for (int e = 0; e < 4 && i + e < n; ++e) dst[i + e] = __uint_as_float(sl[wave][i + e]);
        }
    }
    for (int x = threadIdx.x; x < kDecodeBins; x += 256)
        if (lh[x]) atomicAdd(&dhist[b * kDecodeBins + x], lh[x]);
}

hipError_t launch_decode_append(const Tables &tab, hipStream_t st, int32_t B, const int32_t *cache_len,
                                int64_t ctx_bound, int64_t nblk_cap, const bf16_t *k, const bf16_t *v, const bf16_t *k_idx,
                                const bf16_t *q_idx, bf16_t *k_cache, bf16_t *v_cache, bf16_t *kbar,
                                bf16_t *kpend, bf16_t *qrot, uint32_t *dhist)
{
    hipLaunchKernelGGL(decode_append_kernel, dim3(B), dim3(64), 0, st, tab, cache_len, ctx_bound, nblk_cap, k, v,
                       k_idx, q_idx,
                       k_cache, v_cache, kbar, kpend, qrot, dhist);
    return hipGetLastError();
}

hipError_t launch_token_decode_append(const Tables &tab, hipStream_t st, int32_t B, const int32_t *cache_len,
                                      int64_t ctx_bound, int64_t tok_cap, const bf16_t *k_idx, const bf16_t *q_idx,
                                      bf16_t *ktok, bf16_t *qrot, uint32_t *dhist)
{
    hipLaunchKernelGGL(token_decode_append_kernel, dim3(B), dim3(64), 0, st, tab, cache_len, ctx_bound, tok_cap, k_idx,
                       q_idx, ktok, qrot, dhist);
    return hipGetLastError();
}

hipError_t launch_decode_scan(hipStream_t st, int32_t B, const int32_t *cache_len, int64_t ctx_bound, int rsh,
                              int64_t nblk_cap, int64_t ncol, const bf16_t *qrot, const bf16_t *kbar, float *scores,
                              uint32_t *dhist)
{
    const int64_t o_max = ctx_bound >> rsh;
    if (o_max <= 0) return hipSuccess;
    dim3 grid(static_cast<unsigned>((o_max + kScanBlocksPerWG - 1) / kScanBlocksPerWG), static_cast<unsigned>(B));
    hipLaunchKernelGGL(decode_scan_kernel, grid, dim3(256), 0, st, cache_len, ctx_bound, rsh, nblk_cap, ncol, qrot, kbar,
                       scores, dhist);
    return hipGetLastError();
}

}  // namespace qsa
