// Per-query top-K block selection over a materialised score row (PyTorchKR post
// "Qwen3.8-Flash-Next, 1/9의 학습 비용으로 …", section "QSA: 인덱서 자체의 비용을
// 줄이는 희소 어텐션": token budget K = 2048 with r = 4, i.e. at most 512 blocks
// per query).
//
// Order: score descending, then block index descending (ties go to the more
// recent block).  Scores are >= +0, so their IEEE bit patterns order like the
// values and the K-th largest score is found by an exact MSB-first radix
// select on the 31 value bits (11 + 11 + 9 bits) with LDS histograms.  The
// selected blocks are then emitted in ascending block order by one more pass
// with workgroup-wide prefix counts built from wave ballots.
//
// One workgroup of 256 threads per query row.
#include "qsa_common.h"

namespace qsa {

constexpr int kSelThreads = 256;
constexpr int kSelMaxBins = 2048;

__device__ __forceinline__ uint32_t ballot_count(uint64_t m) { return static_cast<uint32_t>(__popcll(m)); }

__device__ __forceinline__ uint32_t lane_rank(uint64_t m) {
    // number of set bits of m below this lane
    const int lane = threadIdx.x & 63;
    const uint64_t below = (lane == 0) ? 0ull : (m & ((~0ull) >> (64 - lane)));
    return static_cast<uint32_t>(__popcll(below));
}

// Row (b, i), i < L, is the query at position q_offset + i (or cache_len[b]
// clamped to [0, q_offset] when cache_len is given: decode passes its bound); its scores start at scores + b*sc_bstride + i*ncol
// and its selection at block_idx + b*bi_bstride + i*budget.
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    int64_t L, int64_t q_offset, const int32_t *__restrict__ cache_len, int64_t ncol,
    const float *__restrict__ scores, int64_t sc_bstride, int32_t *__restrict__ block_idx, int64_t bi_bstride,
    int budget)
{
    __shared__ uint32_t hist[kSelMaxBins];
    __shared__ uint32_t s_digit, s_above;
    __shared__ uint32_t s_eq[2][4], s_take[2][4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t row = blockIdx.x;
    const int64_t b = row / L;
    const int64_t i = row - b * L;
    const int64_t pos = cache_len ? decode_pos(cache_len, b, q_offset) : q_offset + i;
    const int64_t o = pos / kBlock;
    const uint32_t *srow = reinterpret_cast<const uint32_t *>(scores + b * sc_bstride + i * ncol);
    int32_t *out = block_idx + b * bi_bstride + i * budget;

    if (o <= budget) {
        for (int j = tid; j < budget; j += kSelThreads) out[j] = (j < o) ? j : -1;
        return;
    }

    uint32_t prefix = 0, mask = 0, k_rem = static_cast<uint32_t>(budget), n_eq = 0;
    const int shifts[3] = {20, 9, 0};
    const int nbits[3] = {11, 11, 9};
    for (int r = 0; r < 3; ++r) {
        const int shift = shifts[r];
        const int nb = 1 << nbits[r];
        const uint32_t dmask = static_cast<uint32_t>(nb - 1);
        for (int x = tid; x < nb; x += kSelThreads) hist[x] = 0;
        __syncthreads();
        for (int64_t j = tid; j < o; j += kSelThreads) {
            const uint32_t key = srow[j];
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            const int per = nb / 64;
            const int lo = lane * per;
            uint32_t part = 0;
            for (int d = 0; d < per; ++d) part += hist[lo + d];
            // inclusive suffix sum over lanes: incl = sum of parts of lanes >= lane
            uint32_t incl = part;
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
    // prefix is now the K-th largest score T; n_eq elements equal T and the
    // k_rem of them with the largest block indices are taken.
    const uint32_t T = prefix;
    const uint32_t eq_skip = n_eq - k_rem;     // ties with the smallest indices are dropped

    uint32_t eq_run = 0, take_run = 0;
    int par = 0;
    for (int64_t base = 0; base < o; base += kSelThreads) {
        const int64_t j = base + tid;
        const bool valid = j < o;
        const uint32_t key = valid ? srow[j] : 0u;
        const bool gt = valid && key > T;
        const bool eq = valid && key == T;
        const uint64_t em = __ballot(eq);
        if (lane == 0) s_eq[par][wave] = ballot_count(em);
        __syncthreads();
        uint32_t eq_before = eq_run + lane_rank(em);
        uint32_t eq_tile = 0;
        for (int w = 0; w < 4; ++w) {
            const uint32_t cnt = s_eq[par][w];
            if (w < wave) eq_before += cnt;
            eq_tile += cnt;
        }
        const bool take = gt || (eq && eq_before >= eq_skip);
        const uint64_t tm = __ballot(take);
        if (lane == 0) s_take[par][wave] = ballot_count(tm);
        __syncthreads();
        uint32_t posn = take_run + lane_rank(tm);
        uint32_t take_tile = 0;
        for (int w = 0; w < 4; ++w) {
            const uint32_t cnt = s_take[par][w];
            if (w < wave) posn += cnt;
            take_tile += cnt;
        }
        if (take && posn < static_cast<uint32_t>(budget)) out[posn] = static_cast<int32_t>(j);
        eq_run += eq_tile;
        take_run += take_tile;
        par ^= 1;
    }
}

hipError_t launch_select(hipStream_t st, int32_t B, int64_t L, int64_t q_offset, const int32_t *cache_len,
                         int64_t ncol, const float *scores, int64_t sc_bstride, int32_t *block_idx,
                         int64_t bi_bstride, int budget)
{
    const int64_t rows = static_cast<int64_t>(B) * L;
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(select_kernel, dim3(static_cast<unsigned>(rows)), dim3(kSelThreads), 0, st, L, q_offset,
                       cache_len, ncol, scores, sc_bstride, block_idx, bi_bstride, budget);
    return hipGetLastError();
}

}  // namespace qsa
