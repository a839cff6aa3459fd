// Decode kernels: append one token per sequence and scan the pooled indexer
// keys (PyTorchKR post "Qwen3.8-Flash-Next, 1/9의 학습 비용으로 …", section "QSA:
// 인덱서 자체의 비용을 줄이는 희소 어텐션": the indexer compares the query with the
// mean-pooled, block-start-rotated keys of fully observed blocks, so one
// decode step reads n/4 pooled keys instead of n token keys).
#include <type_traits>

#include "qsa_common.h"

namespace qsa {

constexpr int kDecodeBins = 2048;      // histogram of score bits 30..20

// Append the new token of sequence b at position p, one wave (lane = 0..63):
//   lanes: head g = lane/32, chunk c = lane%32 -> rotate k at p into K~ slot
//          p%4 and copy v into V slot p%4 (when k is given);
//   lanes 0..15: raw k_idx into kpend[p%4]; when p%4 == 3 pool the completed
//          block (kpend slots 0..2 + this token) into kbar[p/4] -- a block
//          that is no candidate of the query at p (candidates are < p/4).
__device__ __forceinline__ void append_one(const Tables &tab, int lane, int64_t b, int64_t p, int64_t nblk_cap,
                                           const bf16_t *__restrict__ k, const bf16_t *__restrict__ v,
                                           const bf16_t *__restrict__ k_idx, bf16_t *__restrict__ k_cache,
                                           bf16_t *__restrict__ v_cache, bf16_t *__restrict__ kbar,
                                           bf16_t *__restrict__ kpend)
{
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
}

// One wave per sequence: append_one at p = cache_len[b] (the step of a reused
// selection, which scores nothing).
__global__ __launch_bounds__(64) void decode_append_kernel(
    Tables tab, const int32_t *__restrict__ cache_len, int64_t ctx_bound, int64_t nblk_cap,
    const bf16_t *__restrict__ k, const bf16_t *__restrict__ v, const bf16_t *__restrict__ k_idx,
    bf16_t *__restrict__ k_cache, bf16_t *__restrict__ v_cache, bf16_t *__restrict__ kbar,
    bf16_t *__restrict__ kpend)
{
    const int64_t b = blockIdx.x;
    append_one(tab, threadIdx.x, b, decode_pos(cache_len, b, ctx_bound), nblk_cap, k, v, k_idx, k_cache, v_cache,
               kbar, kpend);
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

// rotate_chunk8 for a chunk of the rotary dims with its 8 angles' cosines and
// sines already loaded (tc[k], ts[k]: pair j0 + k); first_half: the chunk holds
// dims j of the pairs (j, j + 32), else dims j + 32.
__device__ __forceinline__ u32x4 rotate_chunk8_t(u32x4 x, u32x4 xp, bool first_half, const float (&tc)[8],
                                                 const float (&ts)[8]) {
    uint32_t w[4];
    for (int i = 0; i < 4; ++i) {
        float r[2];
        for (int e = 0; e < 2; ++e) {
            float me = __uint_as_float(e ? (x[i] & 0xFFFF0000u) : (x[i] << 16));
            float pa = __uint_as_float(e ? (xp[i] & 0xFFFF0000u) : (xp[i] << 16));
            float a = first_half ? me : pa, bb = first_half ? pa : me;
            rotate_pair(a, bb, tc[2 * i + e], ts[2 * i + e]);
            r[e] = first_half ? a : bb;
        }
        w[i] = pack_bf16x2(r[0], r[1]);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

// Score scan: scores[b][blk] = sum_h ReLU(<q~_h, k̄_blk>) for blk < floor(p/r),
// r = 1 << rsh (4: pooled micro-blocks; 1: one rotated key per token).
// v_mfma_f32_16x16x32_bf16 with A = q~ (4 real rows of 16), B = 16 keys;
// lanes 0..15 end with the 4 heads of one block.  Each wave streams bpw
// consecutive blocks (chosen per call, up to kScanBlocksPerWaveMax) and collects
// their scores in LDS, then writes them with one 16-byte store per lane and 256
// scores: 4-byte stores interleaved with the k̄ loads cost about 6% of the scan.

// What the first work-group of a sequence appends while the others scan: the
// new token's K~/V (k non-null), its raw indexer key (pooled at r = 4 into the
// key cache when its block completes) or, at r = 1, its indexer key rotated at
// p into the token-key cache.  Nothing appended is read by the scan of the
// same step (candidates are < floor(p/r)).
struct DecodeAppend {
    const bf16_t *k, *v, *k_idx;
    bf16_t *k_cache, *v_cache, *kpend;
    int64_t kv_blk_cap;                  // blocks per sequence and KV group of the K~/V caches
};

// Per-work-group summary of the score histogram.  Work-group w of a row
// writes the bins of its own 2048-bin histogram of score bits 30..20 whose
// count of scores in higher bins (within w) is below the budget K -- the bins
// from the top down to d_w, the highest bin whose suffix count within w
// reaches K, or every bin if w holds fewer than K scores -- as words
// (bin << 21 | count), preceded by their number.  A bin enters only if it is
// non-empty and the higher bins hold fewer than K scores, so at most K words.
// The row's boundary bin d* (the highest bin whose suffix count over the row
// reaches K) is >= every d_w, hence the summaries give the exact row count of
// every bin >= d*: no histogram has to be cleared between steps.

// kList: instead of its scores, each wave stores the list of its scores whose
// digit (bits 30..20) is at or above the lowest digit of its work-group's
// summary -- (score bits, block) pairs in block order, at most bpw of them, in
// cand[((b * nwg + blockIdx.x) * 4 + wave) * bpw ..] with their count in
// candn[(b * nwg + blockIdx.x) * 4 + wave].  The row's boundary digit is at or
// above every work-group's lowest summary digit, so these lists, taken in
// order, hold every score a selection can take.
template <bool kList>
__global__ __launch_bounds__(256) void decode_scan_kernel(Tables tab, const int32_t *__restrict__ cache_len,
                                                          int64_t ctx_bound, int rsh, int64_t key_cap, int64_t ncol,
                                                          int budget, int bpw, int nwg,
                                                          const bf16_t *__restrict__ q_idx,
                                                          bf16_t *__restrict__ keys, float *__restrict__ scores,
                                                          uint32_t *__restrict__ summ, uint2 *__restrict__ cand,
                                                          uint32_t *__restrict__ candn, DecodeAppend ap)
{
    __shared__ uint32_t lh[kDecodeBins];
    __shared__ __attribute__((aligned(16))) uint32_t sl[4][kScanBlocksPerWaveMax];   // each wave's score bits
    __shared__ uint32_t wsum[4];
    __shared__ uint32_t s_low;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t b = blockIdx.y;
    const int64_t p = decode_pos(cache_len, b, ctx_bound);
    const int64_t o = p >> rsh;
    const float *cs = tab.cos + p * kPairs;
    const float *sn = tab.sin + p * kPairs;
    // The row's first wave appends the new token.  With candidates to scan it
    // does so once its first keys are in flight (below), so that the append's
    // round trips overlap that wait; nothing it writes is read by the scan.
    auto append = [&]() {
        if (rsh == 2) {
            append_one(tab, lane, b, p, ap.kv_blk_cap, ap.k, ap.v, ap.k_idx, ap.k_cache, ap.v_cache, keys, ap.kpend);
        } else if (lane < 16) {       // token keys: the new key rotated at p into keys[b][p]
            const bf16_t *src = ap.k_idx + b * kIdxDim;
            const u32x4 x = *reinterpret_cast<const u32x4 *>(src + 8 * lane);
            const u32x4 xp = *reinterpret_cast<const u32x4 *>(src + 8 * (lane ^ 4));
            *reinterpret_cast<u32x4 *>(keys + (b * key_cap + p) * kIdxDim + 8 * lane) =
                rotate_chunk8(x, xp, lane, cs, sn);
        }
    };
    const bool appender = blockIdx.x == 0 && wave == 0;
    if (appender && o == 0) append();
    if (static_cast<int64_t>(blockIdx.x) * 4 * bpw >= o) {           // whole workgroup idle
        if (kList && threadIdx.x < 4) candn[(b * nwg + blockIdx.x) * 4 + threadIdx.x] = 0u;
        return;
    }
    for (int x = threadIdx.x; x < kDecodeBins; x += 256) lh[x] = 0;
    if (threadIdx.x == 0) s_low = 0u;       // (all scores are candidates below the budget)
    __syncthreads();
    const int64_t w0 = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * bpw;
    if (w0 < o) {
    const int r = lane & 15, g = lane >> 4;
    const bf16_t *kb = keys + b * key_cap * kIdxDim;
    const int64_t wend = (w0 + bpw < o) ? w0 + bpw : o;
    // B = 16 blocks of keys per MFMA, 4 MFMAs of 64 blocks per step; blocks
    // past the row (o) read block w0 instead (in bounds, results discarded)
    auto load_step = [&](int64_t c0, bf16x8 (&bf)[4][4]) {
        for (int u = 0; u < 4; ++u) {
            int64_t blk = c0 + 16 * u + r;
            if (blk >= o) blk = w0;
            for (int s = 0; s < 4; ++s)
                bf[u][s] = *reinterpret_cast<const bf16x8 *>(kb + blk * kIdxDim + 32 * s + 8 * g);
        }
    };
    // A = q~: lane (head r < 4, k-group g) holds dims 32s + 8g .. +7 of head r,
    // rotated here at p (pairs j, j + 32 sit in k-steps 0 and 1 of one lane).
    // Its loads go first and the first step's keys right after, so that the
    // rotation waits for the query alone.
    u32x4 x[4];
    float tc[8], ts[8];
    if (r < kIdxHeads) {
        const bf16_t *src = q_idx + (b * kIdxHeads + r) * kIdxDim + 8 * g;
        for (int s = 0; s < 4; ++s) x[s] = *reinterpret_cast<const u32x4 *>(src + 32 * s);
        for (int e = 0; e < 8; ++e) {
            tc[e] = cs[8 * g + e];
            ts[e] = sn[8 * g + e];
        }
    }
    bf16x8 bf[4][4];
    load_step(w0, bf);
    if (appender) append();           // w0 = 0 < o here
    bf16x8 af[4];
    if (r < kIdxHeads) {
        const u32x4 x0 = rotate_chunk8_t(x[0], x[1], true, tc, ts);      // chunk g pairs with chunk g + 4
        const u32x4 x1 = rotate_chunk8_t(x[1], x[0], false, tc, ts);
        af[0] = __builtin_bit_cast(bf16x8, x0);
        af[1] = __builtin_bit_cast(bf16x8, x1);
        af[2] = __builtin_bit_cast(bf16x8, x[2]);
        af[3] = __builtin_bit_cast(bf16x8, x[3]);
    } else {
        for (int s = 0; s < 4; ++s) af[s] = bf16x8{};
    }
    // One step: the 16 MFMAs, then (kNext) the next step's keys into the
    // registers they freed, then the scores of this step into LDS and the
    // histogram -- the loads stay in flight while the scores are stored.
    auto step = [&](int64_t c0, auto next) {
        f32x4 acc[4];
        for (int u = 0; u < 4; ++u) {
            acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < 4; ++s) acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], bf[u][s], acc[u], 0, 0, 0);
        }
        if constexpr (decltype(next)::value) load_step(c0 + 64, bf);
        for (int u = 0; u < 4; ++u) {
            const int64_t blk = c0 + 16 * u + r;
            if (g == 0 && blk < o) {
                float sc = fmaxf(acc[u][0], 0.f) + fmaxf(acc[u][1], 0.f) + fmaxf(acc[u][2], 0.f) + fmaxf(acc[u][3], 0.f);
                const uint32_t bits = __float_as_uint(sc) & 0x7FFFFFFFu;
                sl[wave][blk - w0] = bits;
                atomicAdd(&lh[bits >> 20], 1u);
            }
        }
    };
    int64_t c0 = w0;
    for (; c0 + 64 < wend; c0 += 64) step(c0, std::true_type{});
    step(c0, std::false_type{});
    }
    __syncthreads();
    if (!kList && w0 < o) {   // the wave's scores, blocks w0 .. wend-1
        const int64_t n = ((w0 + bpw < o) ? w0 + bpw : o) - w0;
        float *dst = scores + b * ncol + w0;
        const bool vec = ((b * ncol + w0) & 3) == 0;
        for (int i = 4 * lane; i < n; i += 256) {
            if (vec && i + 3 < n)
                *reinterpret_cast<u32x4 *>(dst + i) = *reinterpret_cast<const u32x4 *>(&sl[wave][i]);
            else
                for (int e = 0; e < 4 && i + e < n; ++e) dst[i + e] = __uint_as_float(sl[wave][i + e]);
        }
    }
    // ---- the work-group's histogram summary: thread t owns bins 8t .. 8t+7
    constexpr int kPer = kDecodeBins / 256;
    uint32_t h[kPer];
    uint32_t part = 0;
    for (int i = 0; i < kPer; ++i) {
        h[i] = lh[threadIdx.x * kPer + i];
        part += h[i];
    }
    uint32_t total;
    const uint32_t below = block_scan_nt<256>(part, wsum, total);       // scores in lower threads' bins
    uint32_t above = total - below - part;                               // scores in higher threads' bins
    uint32_t emit = 0;
    bool take[kPer];
    for (int i = kPer - 1; i >= 0; --i) {
        take[i] = h[i] != 0u && above < static_cast<uint32_t>(budget);
        emit += take[i] ? 1u : 0u;
        // the summary's lowest digit: the one whose count reaches the budget
        if (kList && take[i] && above + h[i] >= static_cast<uint32_t>(budget))
            s_low = static_cast<uint32_t>(threadIdx.x * kPer + i);
        above += h[i];
    }
    uint32_t n_emit;
    uint32_t pos = block_scan_nt<256>(emit, wsum, n_emit);
    uint32_t *slot = summ + (b * nwg + blockIdx.x) * kSumSlot;
    if (threadIdx.x == 0) slot[0] = n_emit;
    for (int i = 0; i < kPer; ++i)
        if (take[i]) slot[1 + pos++] = (static_cast<uint32_t>(threadIdx.x * kPer + i) << 21) | h[i];
    if constexpr (kList) {
        // ---- the candidate list: this wave's scores of digit >= the lowest
        // summary digit (s_low, published by the block scan's barriers), in
        // rounds of 256 blocks (lane l: blocks 4l .. 4l+3 of the round, one
        // 16-byte LDS read), written in block order
        const uint32_t T = s_low << 20;
        const int64_t n = (w0 < o) ? (((w0 + bpw < o) ? w0 + bpw : o) - w0) : 0;
        const int64_t li = (b * nwg + blockIdx.x) * 4 + wave;
        uint2 *dst = cand + li * bpw;
        uint32_t base = 0;
        for (int64_t r0 = 0; r0 < n; r0 += 256) {
            const int64_t i0 = r0 + 4 * lane;
            const u32x4 x = *reinterpret_cast<const u32x4 *>(&sl[wave][i0]);
            bool f[4];
            uint64_t m[4];
            uint32_t before = 0;                 // set flags of lower lanes, all four positions
            for (int j = 0; j < 4; ++j) {
                f[j] = i0 + j < n && x[j] >= T;
                m[j] = __builtin_amdgcn_ballot_w64(f[j]);
                before += lanes_below(m[j]);
            }
            uint32_t own = 0;
            for (int j = 0; j < 4; ++j) {
                if (f[j]) dst[base + before + own] = make_uint2(x[j], static_cast<uint32_t>(w0 + i0 + j));
                own += f[j] ? 1u : 0u;
            }
            for (int j = 0; j < 4; ++j) base += static_cast<uint32_t>(__popcll(m[j]));
        }
        if (lane == 0) candn[li] = base;
    }
}

hipError_t launch_decode_append(const Tables &tab, hipStream_t st, int32_t B, const int32_t *cache_len,
                                int64_t ctx_bound, int64_t nblk_cap, const bf16_t *k, const bf16_t *v, const bf16_t *k_idx,
                                bf16_t *k_cache, bf16_t *v_cache, bf16_t *kbar, bf16_t *kpend)
{
    hipLaunchKernelGGL(decode_append_kernel, dim3(B), dim3(64), 0, st, tab, cache_len, ctx_bound, nblk_cap, k, v,
                       k_idx, k_cache, v_cache, kbar, kpend);
    return hipGetLastError();
}

// Work-groups of the scan per row (the summary slots a row holds).
int64_t decode_scan_wgs(int64_t ncol, int bpw) { return (ncol + 4 * bpw - 1) / (4 * bpw); }

// The scan over rows of at most ncol = ctx_bound >> rsh keys, with the append
// of the new token done by each row's first work-group (a grid of at least one
// work-group per row even when no row has a candidate).
hipError_t launch_decode_scan(const Tables &tab, hipStream_t st, int32_t B, const int32_t *cache_len,
                              int64_t ctx_bound, int rsh, int64_t key_cap, int64_t ncol, int budget, int bpw,
                              const bf16_t *q_idx, bf16_t *keys, float *scores, uint32_t *summ,
                              const bf16_t *k, const bf16_t *v, const bf16_t *k_idx, bf16_t *k_cache,
                              bf16_t *v_cache, bf16_t *kpend, int64_t kv_blk_cap, uint2 *cand, uint32_t *candn)
{
    if (bpw < 64 || bpw > kScanBlocksPerWaveMax || bpw % 64 != 0) return hipErrorInvalidValue;
    const int64_t nwg = decode_scan_wgs(ncol, bpw);
    const DecodeAppend ap{k, v, k_idx, k_cache, v_cache, kpend, kv_blk_cap};
    dim3 grid(static_cast<unsigned>(nwg), static_cast<unsigned>(B));
    if (cand)
        hipLaunchKernelGGL(decode_scan_kernel<true>, grid, dim3(256), 0, st, tab, cache_len, ctx_bound, rsh, key_cap,
                           ncol, budget, bpw, static_cast<int>(nwg), q_idx, keys, scores, summ, cand, candn, ap);
    else
        hipLaunchKernelGGL(decode_scan_kernel<false>, grid, dim3(256), 0, st, tab, cache_len, ctx_bound, rsh, key_cap,
                           ncol, budget, bpw, static_cast<int>(nwg), q_idx, keys, scores, summ, cand, candn, ap);
    return hipGetLastError();
}

}  // namespace qsa
