// Per-query top-K block selection (PyTorchKR post "Qwen3.8-Flash-Next, 1/9의 학습
// 비용으로 …", section "QSA: 인덱서 자체의 비용을 줄이는 희소 어텐션": token budget
// K = 2048 with r = 4, i.e. at most 512 blocks per query).
//
// Order: score descending, then block index descending (ties go to the more
// recent block).  Scores are >= +0, so their IEEE bit patterns order like the
// values and the K-th largest score is found by an exact MSB-first radix
// select on the 31 value bits (11 + 11 + 9 bits) with LDS histograms.  The
// selected blocks are then emitted in ascending block order by one more pass
// with workgroup-wide prefix counts built from wave ballots.  The same routine
// serves three sources of a row's (score, block) sequence, always in ascending
// block order:
//   * a materialised score row (qsa_select, decode),
//   * the compact candidate list a query kept while streaming its scores
//     (the fused index + select path; loaded into LDS first),
//   * scores recomputed on the fly for a query whose candidate list
//     overflowed (exact fallback).
//
// One workgroup of 256 threads per query row.
#include "qsa_common.h"

namespace qsa {

constexpr int kSelThreads = 256;
constexpr int kSelMaxBins = 2048;

__device__ __forceinline__ uint32_t lane_rank(uint64_t m) {
    const int lane = threadIdx.x & 63;
    const uint64_t below = (lane == 0) ? 0ull : (m & ((~0ull) >> (64 - lane)));
    return static_cast<uint32_t>(__popcll(below));
}

// Exact top-`budget` of n > budget keys.  key(j) gives the score bits of
// element j (j ascending = block ascending), id(j) its block.  Writes `budget`
// block ids in ascending order to out.  `hist` is LDS of kSelMaxBins words.
template <int NT = kSelThreads, typename KeyFn, typename IdFn>
__device__ void radix_topk(int64_t n, int budget, KeyFn key, IdFn id, int32_t *__restrict__ out, uint32_t *hist)
{
    constexpr int NW = NT / 64;
    __shared__ uint32_t s_digit, s_above;
    __shared__ uint32_t s_eq[2][NW], s_take[2][NW];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    uint32_t prefix = 0, mask = 0, k_rem = static_cast<uint32_t>(budget), n_eq = 0;
    const int shifts[3] = {20, 9, 0};
    const int nbits[3] = {11, 11, 9};
    for (int r = 0; r < 3; ++r) {
        const int shift = shifts[r];
        const int nb = 1 << nbits[r];
        const uint32_t dmask = static_cast<uint32_t>(nb - 1);
        for (int x = tid; x < nb; x += NT) hist[x] = 0;
        __syncthreads();
        int64_t j = tid;
        for (; j + 3 * NT < n; j += 4 * NT) {        // 4 independent loads in flight
            const uint32_t k0 = key(j), k1 = key(j + NT), k2 = key(j + 2 * NT),
                           k3 = key(j + 3 * NT);
            if ((k0 & mask) == prefix) atomicAdd(&hist[(k0 >> shift) & dmask], 1u);
            if ((k1 & mask) == prefix) atomicAdd(&hist[(k1 >> shift) & dmask], 1u);
            if ((k2 & mask) == prefix) atomicAdd(&hist[(k2 >> shift) & dmask], 1u);
            if ((k3 & mask) == prefix) atomicAdd(&hist[(k3 >> shift) & dmask], 1u);
        }
        for (; j < n; j += NT) {
            const uint32_t k0 = key(j);
            if ((k0 & mask) == prefix) atomicAdd(&hist[(k0 >> shift) & dmask], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            const int per = nb / 64;
            const int lo = lane * per;
            uint32_t part = 0;
            for (int d = 0; d < per; ++d) part += hist[lo + d];
            uint32_t incl = part;                 // sum of parts of lanes >= lane
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t other = __shfl_down(incl, off);
                if (lane + off < 64) incl += other;
            }
            const uint32_t above = incl - part;
            if (above < k_rem && k_rem <= incl) {
                uint32_t acc = above;
                for (int d = per - 1; d >= 0; --d) {
                    const uint32_t h = hist[lo + d];
                    if (acc + h >= k_rem) {
                        s_digit = static_cast<uint32_t>(lo + d);
                        s_above = acc;
                        break;
                    }
                    acc += h;
                }
            }
        }
        __syncthreads();
        const uint32_t digit = s_digit;
        k_rem -= s_above;
        prefix |= digit << shift;
        mask |= dmask << shift;
        n_eq = hist[digit];
        __syncthreads();
    }
    // prefix is the K-th largest score T; n_eq elements equal T and the k_rem
    // of them with the largest block ids (the last ones) are taken.
    const uint32_t T = prefix;
    const uint32_t eq_skip = n_eq - k_rem;

    uint32_t eq_run = 0, take_run = 0;
    int par = 0;
    for (int64_t base = 0; base < n; base += NT) {
        const int64_t j = base + tid;
        const bool valid = j < n;
        const uint32_t k = valid ? key(j) : 0u;
        const bool gt = valid && k > T;
        const bool eq = valid && k == T;
        const uint64_t em = __ballot(eq);
        if (lane == 0) s_eq[par][wave] = static_cast<uint32_t>(__popcll(em));
        __syncthreads();
        uint32_t eq_before = eq_run + lane_rank(em);
        uint32_t eq_tile = 0;
        for (int w = 0; w < NW; ++w) {
            const uint32_t cnt = s_eq[par][w];
            if (w < wave) eq_before += cnt;
            eq_tile += cnt;
        }
        const bool take = gt || (eq && eq_before >= eq_skip);
        const uint64_t tm = __ballot(take);
        if (lane == 0) s_take[par][wave] = static_cast<uint32_t>(__popcll(tm));
        __syncthreads();
        uint32_t posn = take_run + lane_rank(tm);
        uint32_t take_tile = 0;
        for (int w = 0; w < NW; ++w) {
            const uint32_t cnt = s_take[par][w];
            if (w < wave) posn += cnt;
            take_tile += cnt;
        }
        if (take && posn < static_cast<uint32_t>(budget)) out[posn] = static_cast<int32_t>(id(j));
        eq_run += eq_tile;
        take_run += take_tile;
        par ^= 1;
        if (take_run >= static_cast<uint32_t>(budget)) break;     // uniform: every thread saw the same counts
    }
}

// Score of block j for the query whose rotated indexer heads are qs (fp32 [4][128]
// in LDS): sum_h ReLU(<q~_h, k̄_j>), fp32 FMA accumulation (overflow fallback).
__device__ __noinline__ uint32_t recompute_score(const float *qs, const bf16_t *__restrict__ kb, int64_t j)
{
    float d[kIdxHeads] = {0.f, 0.f, 0.f, 0.f};
    const u32x4 *kr = reinterpret_cast<const u32x4 *>(kb + j * kIdxDim);
#pragma unroll 1
    for (int cch = 0; cch < 16; ++cch) {
        const u32x4 w = kr[cch];
        for (int e = 0; e < 8; ++e) {
            const float kv = __uint_as_float(e & 1 ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
            for (int h = 0; h < kIdxHeads; ++h) d[h] = __builtin_fmaf(qs[h * kIdxDim + 8 * cch + e], kv, d[h]);
        }
    }
    const float s = fmaxf(d[0], 0.f) + fmaxf(d[1], 0.f) + fmaxf(d[2], 0.f) + fmaxf(d[3], 0.f);
    return __float_as_uint(s) & 0x7FFFFFFFu;
}

// Copy n 32-bit words from global memory into LDS: 16-byte loads when the
// source is 16-byte aligned, several per thread issued before any store.
template <int NT = kSelThreads>
__device__ __forceinline__ void stage_words(const uint32_t *__restrict__ src, int64_t n, uint32_t *dst)
{
    const int tid = threadIdx.x;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) == 0) {
        const int64_t n4 = n >> 2;
        const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src);
        int64_t j = tid;
        for (; j + 3 * NT < n4; j += 4 * NT) {
            const u32x4 a = s4[j], b = s4[j + NT], c = s4[j + 2 * NT], d = s4[j + 3 * NT];
            reinterpret_cast<u32x4 *>(dst)[j] = a;
            reinterpret_cast<u32x4 *>(dst)[j + NT] = b;
            reinterpret_cast<u32x4 *>(dst)[j + 2 * NT] = c;
            reinterpret_cast<u32x4 *>(dst)[j + 3 * NT] = d;
        }
        for (; j < n4; j += NT) reinterpret_cast<u32x4 *>(dst)[j] = s4[j];
        for (int64_t t = (n4 << 2) + tid; t < n; t += NT) dst[t] = src[t];
    } else {
        int64_t j = tid;
        for (; j + 3 * NT < n; j += 4 * NT) {
            const uint32_t a = src[j], b = src[j + NT], c = src[j + 2 * NT], d = src[j + 3 * NT];
            dst[j] = a; dst[j + NT] = b; dst[j + 2 * NT] = c; dst[j + 3 * NT] = d;
        }
        for (; j < n; j += NT) dst[j] = src[j];
    }
}

__device__ __forceinline__ bool take_all(int64_t o, int budget, int32_t *out) {
    if (o > budget) return false;
    for (int j = threadIdx.x; j < budget; j += blockDim.x) out[j] = (j < o) ? j : -1;
    return true;
}

// Row (b, i), i < L, is the query at position q_offset + i (or cache_len[b]
// clamped to [0, q_offset] when cache_len is given: decode passes its bound); its
// scores start at scores + b*sc_bstride + i*ncol and its selection at
// block_idx + b*bi_bstride + i*budget.
// Rows of up to `lds_words` scores are first staged in (dynamic) LDS so the
// radix passes read on-chip memory; longer rows are read from global memory.
template <int NT>
__global__ __launch_bounds__(NT) void select_kernel(
    int64_t L, int64_t q_offset, const int32_t *__restrict__ cache_len, int64_t ncol,
    const float *__restrict__ scores, int64_t sc_bstride, int32_t *__restrict__ block_idx, int64_t bi_bstride,
    int budget, int64_t lds_words)
{
    __shared__ uint32_t hist[kSelMaxBins];
    extern __shared__ uint32_t rowbuf[];
    const int64_t row = blockIdx.x;
    const int64_t b = row / L;
    const int64_t i = row - b * L;
    const int64_t pos = cache_len ? decode_pos(cache_len, b, q_offset) : q_offset + i;
    const int64_t o = pos / kBlock;
    const uint32_t *srow = reinterpret_cast<const uint32_t *>(scores + b * sc_bstride + i * ncol);
    int32_t *out = block_idx + b * bi_bstride + i * budget;
    if (take_all(o, budget, out)) return;
    if (o <= lds_words) {
        stage_words<NT>(srow, o, rowbuf);
        __syncthreads();
        radix_topk<NT>(o, budget, [&](int64_t j) { return rowbuf[j]; }, [](int64_t j) { return j; }, out, hist);
    } else {
        radix_topk<NT>(o, budget, [&](int64_t j) { return srow[j]; }, [](int64_t j) { return j; }, out, hist);
    }
}

// Workgroup-wide exclusive prefix sum of one value per thread (256 threads).
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *wsum /* LDS [4] */, uint32_t &total)
{
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
    for (int w = 0; w < 4; ++w) {
        if (w < wave) before += wsum[w];
        total += wsum[w];
    }
    __syncthreads();
    return before + incl - v;
}

__device__ __forceinline__ int score_bin(uint32_t bits) {
    const int b = static_cast<int>(bits >> 20) - 951;      // same bins as the fused indexer kernel
    return b < 0 ? 0 : (b > 127 ? 127 : b);
}

// Rows the fused index + select kernel could not finish (a candidate list
// longer than its capacity, or a boundary bin too crowded for its in-LDS
// ranking) are listed in ovf[1 .. ovf[0]] as b*L + i.  Their scores
// I[p][j] = sum_h ReLU(<q~_h, k̄_j>) are recomputed from q~ and k̄ and the
// selection is taken exactly.  Workgroups stride over the list, so the launch
// needs no host-side count.
__global__ __launch_bounds__(kSelThreads) void select_fixup_kernel(
    int64_t L, int64_t q_offset, int rsh, int budget, const int32_t *__restrict__ ovf,
    int32_t *__restrict__ block_idx, int64_t bi_bstride,
    const bf16_t *__restrict__ qrot, int64_t qrot_bstride, const bf16_t *__restrict__ kbar, int64_t nblk_cap)
{
    __shared__ uint32_t hist[kSelMaxBins];
    __shared__ float qs[kIdxHeads * kIdxDim];
    const int tid = threadIdx.x;
    const int n = ovf[0];
    for (int k = blockIdx.x; k < n; k += gridDim.x) {
        const int64_t row = ovf[1 + k];
        const int64_t b = row / L;
        const int64_t i = row - b * L;
        const int64_t o = (q_offset + i) >> rsh;
        int32_t *out = block_idx + b * bi_bstride + i * budget;
        const bf16_t *qr = qrot + b * qrot_bstride + i * kIdxHeads * kIdxDim;
        for (int x = tid; x < kIdxHeads * kIdxDim; x += kSelThreads) qs[x] = bf16_to_f32(qr[x]);
        __syncthreads();
        const bf16_t *kb = kbar + b * nblk_cap * kIdxDim;
        auto score = [&](int64_t j) -> uint32_t { return recompute_score(qs, kb, j); };
        radix_topk(o, budget, score, [](int64_t j) { return j; }, out, hist);
        __syncthreads();
    }
}

// Block-wide exclusive prefix sum for NT threads.

// Decode selection from a score row whose histogram of bits 30..20 (2048
// digits) above the boundary the scan kernel's work-groups already
// summarised: the boundary digit d* and the count above it come from the sum
// of their summaries.  Inside digit d* the high 12 score bits
// are equal, so (low 20 bits, ordinal) is one 32-bit key ordering (score
// desc, block desc).  Rows whose boundary digit holds more than kEqMax scores
// use the plain radix select.
constexpr int kHistNT = 1024;
constexpr int kEqMax = kHistNT;

// Tail of a decode selection, for the kHistNT threads of a workgroup: the
// digit-d* scores (packed keys eqk: low 20 score bits << 10 | ordinal, block
// ids eqb; n_eq of them, in block order) yield the k_rem of rank below k_rem,
// compacted in block order into selq; sel holds the `above` blocks of higher
// digits, ascending; the two lists are merged into out ascending.
__device__ void finish_digit_select(uint32_t *eqk, const int32_t *eqb, const int32_t *sel, int32_t *selq,
                                    uint32_t *wsum, uint32_t n_eq, uint32_t k_rem, uint32_t above, int budget,
                                    int32_t *__restrict__ out)
{
    const int tid = threadIdx.x;
    // digit-d* scores taken: rank < k_rem by key (keys are distinct); their
    // block ids are compacted in block order into selq[0 .. k_rem).  S = 4, 2
    // or 1 adjacent threads share a key, each counting the keys ahead of it in
    // one slice of the list (padded to 128 with zeros, which rank nothing).
    const uint32_t npad = (n_eq + 127) & ~127u;
    for (uint32_t u = n_eq + tid; u < npad; u += kHistNT) eqk[u] = 0u;
    __syncthreads();
    const int S = n_eq <= 256 ? 4 : (n_eq <= 512 ? 2 : 1);
    const uint32_t key_t = static_cast<uint32_t>(tid) / S, slice = static_cast<uint32_t>(tid) % S;
    uint32_t r = 0;
    if (n_eq != k_rem && key_t < n_eq) {
        const uint32_t kx = eqk[key_t];
        const uint32_t per = npad / S;                     // a multiple of 32
        const u32x4 *e4 = reinterpret_cast<const u32x4 *>(eqk + slice * per);
        for (uint32_t u = 0; u < per / 4; u += 8) {
            u32x4 y[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = e4[u + i];
#pragma unroll
            for (int i = 0; i < 8; ++i) r += (y[i][0] > kx) + (y[i][1] > kx) + (y[i][2] > kx) + (y[i][3] > kx);
        }
    }
    if (S >= 2) r += __shfl_xor(r, 1);
    if (S >= 4) r += __shfl_xor(r, 2);
    const bool take = slice == 0 && key_t < n_eq && (n_eq == k_rem || r < k_rem);
    uint32_t ntake;
    const uint32_t qpos = block_scan_nt<kHistNT>(take ? 1u : 0u, wsum, ntake);
    if (take) selq[qpos] = eqb[key_t];
    __syncthreads();
    // merge the two ascending lists sel[0 .. above) and selq[0 .. k_rem)
    const int budget_i = budget;
    if (tid < budget_i) {
        const bool from_gt = static_cast<uint32_t>(tid) < above;
        const int32_t x = from_gt ? sel[tid] : selq[tid - above];
        const int32_t *other = from_gt ? selq : sel;
        uint32_t lo = 0, hi = from_gt ? k_rem : above;        // count of other < x
        while (lo < hi) {
            const uint32_t mid = (lo + hi) >> 1;
            if (other[mid] < x) lo = mid + 1; else hi = mid;
        }
        out[(from_gt ? tid : tid - above) + lo] = x;
    }
}

// Two-stage decode selection, the row's passes spread over many workgroups.
// Stage 1 (select_chunk_kernel): a 256-thread workgroup per kSelChunk scores
// of a row finds the boundary digit d* from the row's histogram, and stores
// its chunk's blocks of digits above d* and its digit-d* (score bits, block)
// pairs, each in block order, with their counts.  Stage 2
// (select_gather_kernel): one workgroup per row concatenates the chunks'
// lists in chunk order (so in block order), ranks the boundary digit's
// scores and merges the two ascending lists.
constexpr int kSelChunk = 4096;
constexpr int kSelChunkMax = kHistNT;       // chunk prefixes are scanned by one workgroup

// Boundary digit of a 2048-bin histogram for NT threads: s_out[0] = d* (the
// highest digit whose suffix count reaches K), s_out[1] = scores above d*.
template <int NT>
__device__ void boundary_digit(const uint32_t *__restrict__ dh, uint32_t K, uint32_t *wsum, uint32_t *s_out)
{
    constexpr int PER = kSelMaxBins / NT;
    const int tid = threadIdx.x;
    uint32_t h[PER];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        h[i] = dh[tid * PER + i];
        sum += h[i];
    }
    uint32_t tot;
    const uint32_t before = block_scan_nt<NT>(sum, wsum, tot);
    uint32_t acc = tot - before - sum;                  // scores in digits above this thread's bins
    if (acc < K && acc + sum >= K) {
        for (int i = PER - 1; i >= 0; --i) {
            if (acc + h[i] >= K) {
                s_out[0] = static_cast<uint32_t>(tid * PER + i);
                s_out[1] = acc;
                break;
            }
            acc += h[i];
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void select_chunk_kernel(
    const int32_t *__restrict__ cache_len, int64_t pos_bound, int rsh, int64_t ncol, const float *__restrict__ scores,
    const uint32_t *__restrict__ summ, int nwg, int bpw, int budget, int nchunk, int32_t *__restrict__ cnt,
    int32_t *__restrict__ gtb, uint32_t *__restrict__ eqs, int32_t *__restrict__ eqi, uint32_t *__restrict__ rowinfo)
{
    __shared__ uint32_t lh[kSelMaxBins];
    __shared__ uint32_t wsum[4];
    __shared__ uint32_t s_dig[2];
    __shared__ uint32_t wcnt[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t b = blockIdx.y;
    const int ch = blockIdx.x;
    const int64_t o = decode_pos(cache_len, b, pos_bound) >> rsh;
    const int64_t c0 = static_cast<int64_t>(ch) * kSelChunk;
    if (o <= budget || c0 >= o) return;                     // whole workgroup
    const int64_t c1 = (c0 + kSelChunk < o) ? c0 + kSelChunk : o;
    const uint32_t *srow = reinterpret_cast<const uint32_t *>(scores + b * ncol);
    // wave w holds scores c0 + 1024w .. +1023, 16 per lane
    uint32_t v[16];
    const int64_t wb = c0 + 1024 * wave;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int64_t j = wb + 64 * u + lane;
        v[u] = (j < c1) ? srow[j] : 0xFFFFFFFFu;          // sentinel: -1 as int32, below every threshold
    }
    // the row's histogram above the boundary, from the scan work-groups' summaries
    for (int x = tid; x < kSelMaxBins; x += 256) lh[x] = 0;
    __syncthreads();
    // 16 threads per summary slot, 16 slots at a time: the slots' reads overlap
    const int64_t nw_b = (o + 4 * bpw - 1) / (4 * bpw);       // work-groups that scanned this row
    for (int64_t w = tid >> 4; w < nw_b; w += 16) {
        const uint32_t *slot = summ + (b * nwg + w) * kSumSlot;
        const uint32_t n = min(slot[0], static_cast<uint32_t>(kSumWords));
        for (uint32_t i = tid & 15; i < n; i += 16) {
            const uint32_t word = slot[1 + i];
            atomicAdd(&lh[word >> 21], word & 0x1FFFFFu);
        }
    }
    __syncthreads();
    boundary_digit<256>(lh, static_cast<uint32_t>(budget), wsum, s_dig);
    const uint32_t dstar = s_dig[0];
    const uint32_t n_eq = lh[dstar];
    const bool store_eq = n_eq <= static_cast<uint32_t>(kEqMax);
    if (ch == 0 && tid == 0) {                              // the row's boundary for stage two
        rowinfo[b * 3] = dstar;
        rowinfo[b * 3 + 1] = s_dig[1];
        rowinfo[b * 3 + 2] = n_eq;
    }
    const int32_t T0 = static_cast<int32_t>(dstar << 20);
    const int32_t T1 = dstar >= 2047u ? INT32_MAX : static_cast<int32_t>((dstar + 1) << 20);
    uint32_t ng = 0, nge = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        ng += static_cast<uint32_t>(__popcll(__builtin_amdgcn_ballot_w64(static_cast<int32_t>(v[u]) >= T1)));
        nge += static_cast<uint32_t>(__popcll(__builtin_amdgcn_ballot_w64(static_cast<int32_t>(v[u]) >= T0)));
    }
    if (lane == 0) {
        wcnt[0][wave] = ng;
        wcnt[1][wave] = nge - ng;
    }
    __syncthreads();
    uint32_t gpos = 0, epos = 0, gtot = 0, etot = 0;
    for (int w = 0; w < 4; ++w) {
        if (w < wave) {
            gpos += wcnt[0][w];
            epos += wcnt[1][w];
        }
        gtot += wcnt[0][w];
        etot += wcnt[1][w];
    }
    const int64_t slot = b * nchunk + ch;
    int32_t *g_out = gtb + slot * kMaxBudget;
    uint32_t *e_bits = eqs + slot * kEqMax;
    int32_t *e_ids = eqi + slot * kEqMax;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const bool ge = static_cast<int32_t>(v[u]) >= T0;
        const uint64_t gem = __builtin_amdgcn_ballot_w64(ge);
        if (gem == 0) continue;                                  // wave-uniform
        const bool g = static_cast<int32_t>(v[u]) >= T1;
        const uint64_t gm = __builtin_amdgcn_ballot_w64(g);
        const uint64_t em = gem & ~gm;
        const int32_t blk = static_cast<int32_t>(wb + 64 * u + lane);
        if (g) {
            const uint32_t t = gpos + lanes_below(gm);
            if (t < static_cast<uint32_t>(kMaxBudget)) g_out[t] = blk;
        } else if (ge && store_eq) {
            const uint32_t t = epos + lanes_below(em);
            if (t < static_cast<uint32_t>(kEqMax)) {
                e_bits[t] = v[u];
                e_ids[t] = blk;
            }
        }
        gpos += static_cast<uint32_t>(__popcll(gm));
        epos += static_cast<uint32_t>(__popcll(em));
    }
    if (tid == 0) {
        cnt[slot * 2] = static_cast<int32_t>(gtot);
        cnt[slot * 2 + 1] = static_cast<int32_t>(etot);
    }
}

// Largest c in [0, n) with pre[c] <= t (pre ascending, pre[0] = 0).
__device__ __forceinline__ int chunk_of(const uint32_t *pre, int n, uint32_t t) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(kHistNT) void select_gather_kernel(
    const int32_t *__restrict__ cache_len, int64_t pos_bound, int rsh, int64_t ncol, const float *__restrict__ scores,
    const uint32_t *__restrict__ rowinfo, int nchunk, const int32_t *__restrict__ cnt, const int32_t *__restrict__ gtb,
    const uint32_t *__restrict__ eqs, const int32_t *__restrict__ eqi, int32_t *__restrict__ block_idx, int budget)
{
    constexpr int NW = kHistNT / 64;
    __shared__ uint32_t hist[kSelMaxBins];
    __shared__ __attribute__((aligned(16))) uint32_t eqk[kEqMax];
    __shared__ int32_t eqb[kEqMax];
    __shared__ int32_t sel[kMaxBudget];
    __shared__ int32_t selq[kMaxBudget];
    __shared__ uint32_t wsum[NW];
    __shared__ uint32_t gpre[kSelChunkMax], epre[kSelChunkMax];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int64_t o = decode_pos(cache_len, b, pos_bound) >> rsh;
    int32_t *out = block_idx + b * budget;
    if (take_all(o, budget, out)) return;
    const uint32_t above = rowinfo[b * 3 + 1];
    const uint32_t k_rem = static_cast<uint32_t>(budget) - above;
    const uint32_t n_eq = rowinfo[b * 3 + 2];
    if (n_eq > static_cast<uint32_t>(kEqMax)) {
        const uint32_t *srow = reinterpret_cast<const uint32_t *>(scores + b * ncol);
        radix_topk<kHistNT>(o, budget, [&](int64_t j) { return srow[j]; }, [](int64_t j) { return j; }, out, hist);
        return;
    }
    const int nch = static_cast<int>((o + kSelChunk - 1) / kSelChunk);
    const int64_t slot0 = b * nchunk;
    const uint32_t cg = tid < nch ? static_cast<uint32_t>(cnt[(slot0 + tid) * 2]) : 0u;
    const uint32_t ce = tid < nch ? static_cast<uint32_t>(cnt[(slot0 + tid) * 2 + 1]) : 0u;
    uint32_t tg, te;
    const uint32_t pg = block_scan_nt<kHistNT>(cg, wsum, tg);
    const uint32_t pe = block_scan_nt<kHistNT>(ce, wsum, te);
    if (tid < nch) {
        gpre[tid] = pg;
        epre[tid] = pe;
    }
    __syncthreads();
    // concatenate the chunks' lists in chunk (= block) order
    if (static_cast<uint32_t>(tid) < above) {
        const int c = chunk_of(gpre, nch, static_cast<uint32_t>(tid));
        sel[tid] = gtb[(slot0 + c) * kMaxBudget + (tid - gpre[c])];
    }
    if (static_cast<uint32_t>(tid) < n_eq) {
        const int c = chunk_of(epre, nch, static_cast<uint32_t>(tid));
        const int64_t e = (slot0 + c) * kEqMax + (tid - epre[c]);
        eqk[tid] = ((eqs[e] & 0xFFFFFu) << 10) | static_cast<uint32_t>(tid);
        eqb[tid] = eqi[e];
    }
    __syncthreads();
    finish_digit_select(eqk, eqb, sel, selq, wsum, n_eq, k_rem, above, budget, out);
}

// Decode selection from the scan's candidate lists (rows scanned by at most
// kListMaxWG work-groups): one 1,024-thread work-group per row.  The row's
// boundary digit d* and the count above it come from the scan's summaries;
// the lists (one per scan wave), concatenated in order, hold the row's scores
// of digit >= each work-group's lowest summary digit in block order, hence
// every score of digit >= d*.  Blocks above d* are taken, the digit-d* entries ranked by
// (low score bits, ordinal) and the two ascending lists merged, as in the
// two-stage path; a crowded boundary digit (or more candidates than the
// fast path holds) uses the exact radix select over the candidates.
constexpr int kListMaxWG = 8;
constexpr int kListPerLane = 16;          // fast path: up to 16 candidates per thread

__global__ __launch_bounds__(kHistNT) void select_list_kernel(
    const int32_t *__restrict__ cache_len, int64_t pos_bound, int rsh, const uint32_t *__restrict__ summ, int nwg,
    int bpw, const uint2 *__restrict__ cand, const uint32_t *__restrict__ candn, int32_t *__restrict__ block_idx,
    int budget)
{
    constexpr int NW = kHistNT / 64;
    __shared__ uint32_t hist[kSelMaxBins];
    __shared__ __attribute__((aligned(16))) uint32_t eqk[kEqMax];
    __shared__ int32_t eqb[kEqMax];
    __shared__ int32_t sel[kMaxBudget];
    __shared__ int32_t selq[kMaxBudget];
    __shared__ uint32_t wsum[NW];
    __shared__ uint32_t wcnt[2][NW];
    __shared__ uint32_t s_dig[2];
    __shared__ uint32_t pre[4 * kListMaxWG + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t b = blockIdx.x;
    const int64_t o = decode_pos(cache_len, b, pos_bound) >> rsh;
    int32_t *out = block_idx + b * budget;
    if (take_all(o, budget, out)) return;
    const int64_t cap = bpw;                                   // entries per wave's list
    const int nw_b = static_cast<int>((o + 4 * cap - 1) / (4 * cap));   // <= nwg <= kListMaxWG (checked by the launcher)
    const int nl = 4 * nw_b;                                   // the row's lists, one per scan wave, in block order
    // list lengths (lanes 0 .. nl-1 of wave 0) and their prefix
    if (wave == 0) {
        const uint32_t c = lane < nl ? candn[b * nwg * 4 + lane] : 0u;
        uint32_t incl = c;
        for (int off = 1; off <= 4 * kListMaxWG; off <<= 1) {        // lanes 0 .. 4*kListMaxWG
            const uint32_t x = __shfl_up(incl, off);
            if (lane >= off) incl += x;
        }
        if (lane <= nl) pre[lane] = incl - c;                  // pre[nl] = the total
    }
    for (int x = tid; x < kSelMaxBins; x += kHistNT) hist[x] = 0;
    __syncthreads();
    const uint32_t n_c = pre[nl];
    const uint2 *crow = cand + b * nwg * 4 * cap;
    auto cand_at = [&](int64_t j) -> uint2 {
        const int w = chunk_of(pre, nl, static_cast<uint32_t>(j));
        return crow[w * cap + (j - pre[w])];
    };
    // the candidates this thread classifies (wave w: w*S .. w*S + S-1, S a
    // multiple of 64), loaded before the summaries so both round trips overlap
    const uint32_t S = ((n_c + NW * 64 - 1) / (NW * 64)) * 64;
    const bool fast = n_c <= static_cast<uint32_t>(kHistNT * kListPerLane);
    uint2 v[kListPerLane];
#pragma unroll
    for (int u = 0; u < kListPerLane; ++u) {
        const uint32_t j = wave * S + 64 * u + lane;
        v[u] = (fast && 64u * u < S && j < n_c) ? cand_at(j) : make_uint2(0xFFFFFFFFu, 0u);
    }
    // the row's histogram at and above the boundary, from the summaries: 16
    // threads per slot, each slot's first 8 words per thread loaded with its count
    for (int w = tid >> 4; w < nw_b; w += kHistNT / 16) {
        const uint32_t *slot = summ + (b * nwg + w) * kSumSlot;
        const uint32_t i0 = tid & 15;
        uint32_t word[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) word[k] = slot[1 + i0 + 16 * k];
        const uint32_t n = min(slot[0], static_cast<uint32_t>(kSumWords));
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (i0 + 16 * k < n) atomicAdd(&hist[word[k] >> 21], word[k] & 0x1FFFFFu);
        for (uint32_t i = i0 + 128; i < n; i += 16) {
            const uint32_t wd = slot[1 + i];
            atomicAdd(&hist[wd >> 21], wd & 0x1FFFFFu);
        }
    }
    __syncthreads();
    boundary_digit<kHistNT>(hist, static_cast<uint32_t>(budget), wsum, s_dig);
    const uint32_t dstar = s_dig[0];
    const uint32_t above = s_dig[1];
    const uint32_t n_eq = hist[dstar];
    const uint32_t k_rem = static_cast<uint32_t>(budget) - above;
    if (n_eq > static_cast<uint32_t>(kEqMax) || !fast || n_c <= static_cast<uint32_t>(budget)) {
        __syncthreads();                               // every thread has read hist[dstar]
        if (n_c <= static_cast<uint32_t>(budget)) {    // (cannot happen: the lists hold >= budget scores)
            for (uint32_t t = tid; t < static_cast<uint32_t>(budget); t += kHistNT)
                out[t] = (t < n_c) ? static_cast<int32_t>(cand_at(t).y) : -1;
            return;
        }
        radix_topk<kHistNT>(n_c, budget, [&](int64_t j) { return cand_at(j).x; },
                            [&](int64_t j) { return static_cast<int64_t>(cand_at(j).y); }, out, hist);
        return;
    }
    const int32_t T0 = static_cast<int32_t>(dstar << 20);
    const int32_t T1 = dstar >= 2047u ? INT32_MAX : static_cast<int32_t>((dstar + 1) << 20);
    uint32_t ng = 0, nge = 0;
#pragma unroll
    for (int u = 0; u < kListPerLane; ++u) {
        ng += static_cast<uint32_t>(__popcll(__builtin_amdgcn_ballot_w64(static_cast<int32_t>(v[u].x) >= T1)));
        nge += static_cast<uint32_t>(__popcll(__builtin_amdgcn_ballot_w64(static_cast<int32_t>(v[u].x) >= T0)));
    }
    if (lane == 0) {
        wcnt[0][wave] = ng;
        wcnt[1][wave] = nge - ng;
    }
    __syncthreads();
    uint32_t gpos = 0, epos = 0, gtot = 0, etot = 0;
    for (int w = 0; w < NW; ++w) {
        if (w < wave) {
            gpos += wcnt[0][w];
            epos += wcnt[1][w];
        }
        gtot += wcnt[0][w];
        etot += wcnt[1][w];
    }
    if (gtot != above || etot != n_eq) {               // the lists disagree with the summaries: exact path
        radix_topk<kHistNT>(n_c, budget, [&](int64_t j) { return cand_at(j).x; },
                            [&](int64_t j) { return static_cast<int64_t>(cand_at(j).y); }, out, hist);
        return;
    }
#pragma unroll
    for (int u = 0; u < kListPerLane; ++u) {
        const bool ge = static_cast<int32_t>(v[u].x) >= T0;
        const uint64_t gem = __builtin_amdgcn_ballot_w64(ge);
        if (gem == 0) continue;                                  // wave-uniform
        const bool g = static_cast<int32_t>(v[u].x) >= T1;
        const uint64_t gm = __builtin_amdgcn_ballot_w64(g);
        const uint64_t em = gem & ~gm;
        if (g) sel[gpos + lanes_below(gm)] = static_cast<int32_t>(v[u].y);
        if (ge && !g) {
            const uint32_t t = epos + lanes_below(em);
            eqk[t] = ((v[u].x & 0xFFFFFu) << 10) | t;
            eqb[t] = static_cast<int32_t>(v[u].y);
        }
        gpos += static_cast<uint32_t>(__popcll(gm));
        epos += static_cast<uint32_t>(__popcll(em));
    }
    __syncthreads();
    finish_digit_select(eqk, eqb, sel, selq, wsum, n_eq, k_rem, above, budget, out);
}

hipError_t launch_select_list(hipStream_t st, int32_t B, const int32_t *cache_len, int64_t pos_bound, int rsh,
                              const uint32_t *summ, int nwg, int bpw, const uint2 *cand, const uint32_t *candn,
                              int32_t *block_idx, int budget)
{
    if (B <= 0) return hipSuccess;
    if (nwg > kListMaxWG) return hipErrorInvalidValue;
    hipLaunchKernelGGL(select_list_kernel, dim3(static_cast<unsigned>(B)), dim3(kHistNT), 0, st, cache_len, pos_bound,
                       rsh, summ, nwg, bpw, cand, candn, block_idx, budget);
    return hipGetLastError();
}

hipError_t launch_select_two_stage(hipStream_t st, int32_t B, const int32_t *cache_len, int64_t pos_bound, int rsh,
                                   int64_t ncol, const float *scores, const uint32_t *summ, int nwg, int bpw, int32_t *cnt,
                                   int32_t *gtb, uint32_t *eqs, int32_t *eqi, uint32_t *rowinfo, int32_t *block_idx,
                                   int budget)
{
    if (B <= 0) return hipSuccess;
    const int64_t nchunk = (ncol + kSelChunk - 1) / kSelChunk;
    if (nchunk > kSelChunkMax) return hipErrorInvalidValue;
    hipLaunchKernelGGL(select_chunk_kernel, dim3(static_cast<unsigned>(nchunk), static_cast<unsigned>(B)), dim3(256),
                       0, st, cache_len, pos_bound, rsh, ncol, scores, summ, nwg, bpw, budget, static_cast<int>(nchunk), cnt,
                       gtb, eqs, eqi, rowinfo);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(select_gather_kernel, dim3(static_cast<unsigned>(B)), dim3(kHistNT), 0, st, cache_len, pos_bound,
                       rsh, ncol, scores, rowinfo, static_cast<int>(nchunk), cnt, gtb, eqs, eqi, block_idx, budget);
    return hipGetLastError();
}

hipError_t launch_select(hipStream_t st, int32_t B, int64_t L, int64_t q_offset, const int32_t *cache_len,
                         int64_t ncol, const float *scores, int64_t sc_bstride, int32_t *block_idx,
                         int64_t bi_bstride, int budget)
{
    const int64_t rows = static_cast<int64_t>(B) * L;
    if (rows == 0) return hipSuccess;
    // stage rows in LDS when one row fits beside the histogram (up to 36,864 scores)
    const int64_t lds_words = (ncol <= 36864) ? ncol : 0;
    const size_t dyn = static_cast<size_t>(lds_words) * 4;
    // few long rows (decode): 1024 threads per row; many rows: 256
    const bool wide = rows < 1024;
    static thread_local int lds_limit_set = 0;      // per thread: attribute calls are not stream-ordered
    if (dyn > 64 * 1024 && !lds_limit_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(select_kernel<256>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 36864 * 4);
        if (e == hipSuccess)
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(select_kernel<1024>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, 36864 * 4);
        if (e != hipSuccess) return e;
        lds_limit_set = 1;
    }
    if (wide)
        hipLaunchKernelGGL(select_kernel<1024>, dim3(static_cast<unsigned>(rows)), dim3(1024), dyn, st, L, q_offset,
                           cache_len, ncol, scores, sc_bstride, block_idx, bi_bstride, budget, lds_words);
    else
        hipLaunchKernelGGL(select_kernel<256>, dim3(static_cast<unsigned>(rows)), dim3(256), dyn, st, L, q_offset,
                           cache_len, ncol, scores, sc_bstride, block_idx, bi_bstride, budget, lds_words);
    return hipGetLastError();
}

hipError_t launch_select_fixup(hipStream_t st, int32_t B, int64_t L, int64_t q_offset, int rsh, int budget,
                               const int32_t *ovf, int32_t *block_idx, int64_t bi_bstride, const bf16_t *qrot,
                               int64_t qrot_bstride, const bf16_t *kbar, int64_t nblk_cap)
{
    const int64_t rows = static_cast<int64_t>(B) * L;
    if (rows == 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>(rows < 512 ? rows : 512);
    hipLaunchKernelGGL(select_fixup_kernel, dim3(grid), dim3(kSelThreads), 0, st, L, q_offset, rsh, budget, ovf, block_idx,
                       bi_bstride, qrot, qrot_bstride, kbar, nblk_cap);
    return hipGetLastError();
}

}  // namespace qsa
