// Indexer score kernel: I[p][b] = sum_h ReLU(<q~_h(p), k̄_b>) for every
// candidate block b < floor(p/4) (PyTorchKR post "Qwen3.8-Flash-Next, 1/9의
// 학습 비용으로 …", section "QSA: 인덱서 자체의 비용을 줄이는 희소 어텐션", equation
// I_ib; block-causal: only fully observed blocks are scored).
//
// GEMM view: M = 4 * queries (the 4 indexer heads of a query on 4 consecutive
// rows), N = blocks, K = 128.  bf16 operands, fp32 accumulation on the matrix
// cores (v_mfma_f32_32x32x16_bf16).  In the 32x32 accumulator layout each lane
// holds 4 consecutive rows of one column per row group, i.e. the 4 heads of
// one query against one block, so the ReLU + head sum stays inside the lane.
//
// Work decomposition: a workgroup (4 waves) owns 64 queries x up to 512
// blocks.  Each wave keeps its 16 queries' rotated indexer queries (2 A tiles
// of 32 rows) in registers for the whole column range; k̄ tiles of 64 blocks
// are staged through LDS (double buffered) and shared by the 4 waves.
// Workgroups whose column range lies wholly past the causal limit of their
// queries exit at once (causal tile skipping).
#include <type_traits>

#include "qsa_common.h"

namespace qsa {

constexpr int kIdxQueriesPerWG = 64;
constexpr int kIdxColsPerWG = 512;
constexpr int kIdxSubCols = 64;
constexpr int kLdsRow = kIdxDim + 8;   // padded row (elements) against bank conflicts

// ReLU as a clamp to [0, FLT_MAX] (v_med3_f32): one instruction, no NaN
// canonicalisation (inputs are finite).  May return -0 for -0.
__device__ __forceinline__ float relu_fast(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, 3.402823466e38f); }
__device__ __forceinline__ float relu_sum4_fast(float a, float b, float c, float d) {
    return (relu_fast(a) + relu_fast(b)) + (relu_fast(c) + relu_fast(d));
}

__device__ __forceinline__ float relu_sum4(float a, float b, float c, float d) {
    float s = fmaxf(a, 0.0f) + fmaxf(b, 0.0f) + fmaxf(c, 0.0f) + fmaxf(d, 0.0f);
    return __uint_as_float(__float_as_uint(s) & 0x7FFFFFFFu);   // +0 for an all-clipped block
}

// Queries i = 0..L-1 of each sequence sit at positions q_offset + i; their
// rotated indexer queries are at qrot + b*qrot_bstride + i*512 and their score
// rows at scores + b*sc_bstride + i*ncol.
__global__ __launch_bounds__(256) void indexer_scores_kernel(
    int64_t L, int64_t q_offset, int64_t ncol, int64_t nblk_cap,
    const bf16_t *__restrict__ qrot, int64_t qrot_bstride,
    const bf16_t *__restrict__ kbar,      // [B][nblk_cap][128]
    float *__restrict__ scores, int64_t sc_bstride,
    int fill_noncand)
{
    __shared__ __attribute__((aligned(16))) bf16_t lds[2][kIdxSubCols * kLdsRow];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t b = blockIdx.z;
    const int64_t q0 = static_cast<int64_t>(blockIdx.y) * kIdxQueriesPerWG;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kIdxColsPerWG;
    const int64_t q_last = (q0 + kIdxQueriesPerWG - 1 < L) ? q0 + kIdxQueriesPerWG - 1 : L - 1;
    const int64_t o_hi = (q_offset + q_last) / kBlock;         // candidates of the latest query
    const int64_t c_lim = (c0 + kIdxColsPerWG < ncol) ? c0 + kIdxColsPerWG : ncol;
    const int64_t c_end = (o_hi < c_lim) ? o_hi : c_lim;       // columns with any candidate

    float *srow_base = scores + b * sc_bstride;

    // Non-candidate fill (only when the caller wants the full score matrix).
    if (fill_noncand) {
        for (int64_t qq = q0 + wave; qq <= q_last; qq += 4) {
            const int64_t o = (q_offset + qq) / kBlock;
            const int64_t from = (o > c0) ? o : c0;
            for (int64_t c = from + lane; c < c_lim; c += 64) srow_base[qq * ncol + c] = -1.0f;
        }
    }
    if (c0 >= c_end) return;

    // A fragments: wave rows [64*wave, 64*wave+64) of the tile; tile a covers 32 rows.
    bf16x8 afrag[2][8];
    for (int a = 0; a < 2; ++a) {
        const int r = 64 * wave + 32 * a + (lane & 31);         // row = 4*query + head
        const int64_t q = q0 + (r >> 2);
        const int h = r & 3;
        for (int s = 0; s < 8; ++s) {
            if (q < L) {
                const bf16_t *src = qrot + b * qrot_bstride + (q * kIdxHeads + h) * kIdxDim + 16 * s + 8 * (lane >> 5);
                afrag[a][s] = *reinterpret_cast<const bf16x8 *>(src);
            } else {
                afrag[a][s] = bf16x8{};
            }
        }
    }

    const bf16_t *kb = kbar + b * nblk_cap * kIdxDim;
    auto stage = [&](int buf, int64_t cs) {
        // 64 rows x 256 B = 1024 chunks of 16 B; 256 threads x 4
        for (int it = 0; it < 4; ++it) {
            const int chunk = it * 256 + tid;
            const int row = chunk >> 4, c = chunk & 15;
            const int64_t blk = cs + row;
            u32x4 val = u32x4{0, 0, 0, 0};
            if (blk < nblk_cap) val = *reinterpret_cast<const u32x4 *>(kb + blk * kIdxDim + 8 * c);
            *reinterpret_cast<u32x4 *>(&lds[buf][row * kLdsRow + 8 * c]) = val;
        }
    };

    int buf = 0;
    stage(0, c0);
    __syncthreads();
    for (int64_t cs = c0; cs < c_end; cs += kIdxSubCols) {
        if (cs + kIdxSubCols < c_end) stage(buf ^ 1, cs + kIdxSubCols);

        f32x16 acc[2][2];
        for (int ct = 0; ct < 2; ++ct) {
            bf16x8 bfrag[8];
            const bf16_t *brow = &lds[buf][(32 * ct + (lane & 31)) * kLdsRow + 8 * (lane >> 5)];
            for (int s = 0; s < 8; ++s) bfrag[s] = *reinterpret_cast<const bf16x8 *>(brow + 16 * s);
            for (int a = 0; a < 2; ++a) {
                f32x16 c = {};
                for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[a][s], bfrag[s], c, 0, 0, 0);
                acc[a][ct] = c;
            }
        }
        // Epilogue: lane holds, for row group i, the 4 heads of query 2i + lane/32
        // (of the 8 queries of the A tile) against column lane%32.
        for (int a = 0; a < 2; ++a) {
            for (int ct = 0; ct < 2; ++ct) {
                const int64_t col = cs + 32 * ct + (lane & 31);
                for (int i = 0; i < 4; ++i) {
                    const int64_t q = q0 + 16 * wave + 8 * a + 2 * i + (lane >> 5);
                    if (q >= L || col >= ncol) continue;
                    const f32x16 &c = acc[a][ct];
                    const float s = relu_sum4(c[4 * i], c[4 * i + 1], c[4 * i + 2], c[4 * i + 3]);
                    const int64_t o = (q_offset + q) / kBlock;
                    if (col < o) srow_base[q * ncol + col] = s;
                }
            }
        }
        __syncthreads();
        buf ^= 1;
    }
}

hipError_t launch_indexer_scores(hipStream_t st, int32_t B, int64_t L, int64_t q_offset, int64_t ncol,
                                 int64_t nblk_cap, const bf16_t *qrot, int64_t qrot_bstride, const bf16_t *kbar,
                                 float *scores, int64_t sc_bstride, bool fill_noncand)
{
    if (L <= 0 || ncol <= 0) return hipSuccess;
    dim3 grid(static_cast<unsigned>((ncol + kIdxColsPerWG - 1) / kIdxColsPerWG),
              static_cast<unsigned>((L + kIdxQueriesPerWG - 1) / kIdxQueriesPerWG), static_cast<unsigned>(B));
    hipLaunchKernelGGL(indexer_scores_kernel, grid, dim3(256), 0, st, L, q_offset, ncol, nblk_cap, qrot,
                       qrot_bstride, kbar, scores, sc_bstride, fill_noncand ? 1 : 0);
    return hipGetLastError();
}



// ----------------------------------------------------------------------------
// Fused indexer + streaming candidate filter (the index + select stage without
// a score matrix).
//
// A workgroup owns 64 consecutive queries and walks every candidate column
// 0 .. floor(p_last/r) in k̄ tiles of 64, computing the same MFMA scores as
// indexer_scores_kernel.  r = 1 << rsh is the compression ratio: 4 for QSA's
// pooled micro-blocks, 1 for the token-level indexer it is compared against
// (one rotated key per token, candidates t < p).  Each query keeps
//   * a running threshold tau (fp32), below which a block can no longer be in
//     its top `budget`: tau is the lower edge of the highest bin of a 128-bin
//     log histogram (8 bins per octave over [2^-8, 2^8)) of the scores kept so
//     far whose suffix count reaches `budget` -- at least `budget` kept scores
//     are >= tau, so the budget-th largest score is >= tau;
//   * the list of (score, block) pairs with score >= tau, appended in ascending
//     block order (ballot + prefix count per 32-column tile).
// Queries are owned by one wave each, so the histograms, counters and
// thresholds need no workgroup barrier.  After the last tile each wave takes
// its queries' exact top-`budget` from their lists: every kept score in a bin
// above the boundary bin (the highest bin whose suffix count reaches `budget`)
// is selected, and the rest come from the boundary bin, ranked in LDS.  Both
// parts keep the list's (ascending) block order, so one bitonic merge writes
// the selection in ascending block order.  A list that outgrew `cap`
// (it keeps counting without storing) or a boundary bin too crowded to rank
// here sends its row to select_fixup_kernel, which recomputes it exactly.
// Workgroups are issued latest-queries-first (longest rows first).
constexpr int kTopkBins = 128;
constexpr int kTopkBinBase = 951;      // bin 1 = [2^-8, 2^-8 * 1.125); 952 = (127 - 8) * 8

__device__ __forceinline__ int topk_bin(float s) {
    const int b = static_cast<int>(__float_as_uint(s) >> 20) - kTopkBinBase;
    return b < 0 ? 0 : (b >= kTopkBins ? kTopkBins - 1 : b);
}
// Bits of the lower edge of the bin above threshold t (a bin edge or +inf):
// kept scores with bits >= it lie above t's bin; none lies above the top bin.
__device__ __forceinline__ uint32_t next_bin_bits(float t) {
    const uint32_t tb = __float_as_uint(t);
    if (tb == 0u) return static_cast<uint32_t>(kTopkBinBase + 1) << 20;
    return tb >= (static_cast<uint32_t>(kTopkBinBase + kTopkBins - 1) << 20) ? 0x7F800000u : tb + (1u << 20);
}
__device__ __forceinline__ float topk_bin_edge(int b) {
    return b <= 0 ? 0.0f : __uint_as_float(static_cast<uint32_t>(b + kTopkBinBase) << 20);
}

constexpr int kTopkBMax = 1536;        // boundary-bin entries a wave ranks in LDS
constexpr int kTopkRankMax = 512;      // clamped end bins: ranked by counting up to this many
constexpr int kU = 32;                 // list entries per lane in flight in the final pass

// Which of nb packed boundary keys (nb <= 64*R; the low 11 bits of a key are
// its ordinal) are among the k_rem largest, 0 < k_rem < nb: afterwards
// bkey[t] is 1 for those ordinals and 0 for the others.  Padding keys are 0: a
// real key is 0 only for ordinal 0 with equal low score bits, the smallest
// real key, so every rank below k_rem < nb holds a real key.
template <int R>
__device__ __forceinline__ void boundary_mark(uint32_t *bkey, uint32_t nb, uint32_t k_rem, int lane) {
    uint32_t k[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t i = r * 64 + lane;
        k[r] = (i < nb) ? bkey[i] : 0u;
        if (i < nb) bkey[i] = 0u;                 // the same lane's read came first
    }
    wave_sort_desc<R>(k, lane);
    wave_sync();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t i = lane * R + r;
        if (i < k_rem) bkey[k[r] & 0x7FFu] = 1u;
    }
}

// Write n (<= 64*R) block ids to out[] ascending, given as two ascending runs
// sel[0 .. above) and sel[above .. n) of distinct ids: the first run followed
// by the second reversed (then 0 padding) is bitonic, so the last merge phase
// of the wave's bitonic network (log2(64 R) steps) orders it.
template <int R>
__device__ __forceinline__ void emit_merged(const int32_t *sel, int above, int n, int32_t *__restrict__ out, int lane) {
    uint32_t k[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int e = lane * R + r;
        const int src = e < above ? e : n - 1 - e + above;
        k[r] = (e < n) ? static_cast<uint32_t>(sel[src]) + 1u : 0u;    // ids + 1 sort ahead of the padding
    }
    bitonic_steps<R, 64 * R, 32 * R>(k, lane);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = lane * R + r;
        if (i < n) out[n - 1 - i] = static_cast<int32_t>(k[r] - 1u);
    }
}

__global__ __launch_bounds__(256, 2) void indexer_topk_kernel(
    int64_t L, int64_t q_offset, int rsh, int64_t nblk_cap, int budget, int cap,
    const bf16_t *__restrict__ qrot, int64_t qrot_bstride, const bf16_t *__restrict__ kbar,
    uint2 *__restrict__ cand, int32_t *__restrict__ bidx, int64_t bi_bstride, int32_t *__restrict__ ovf)
{
    __shared__ __attribute__((aligned(16))) bf16_t lds[2][kIdxSubCols * kLdsRow];
    __shared__ uint32_t hist[kIdxQueriesPerWG][kTopkBins];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const uint32_t bit = 1u << (lane & 31);
    const int64_t b = blockIdx.y;
    const int64_t tile = static_cast<int64_t>(gridDim.x) - 1 - blockIdx.x;
    const int64_t q0 = tile * kIdxQueriesPerWG;
    const int64_t q_last = (q0 + kIdxQueriesPerWG - 1 < L) ? q0 + kIdxQueriesPerWG - 1 : L - 1;
    const int64_t o_hi = (q_offset + q_last) >> rsh;
    if (o_hi <= budget) {                       // every row of the tile keeps all its candidates
        for (int64_t q = q0 + wave; q <= q_last; q += 4) {
            const int64_t o = (q_offset + q) >> rsh;
            int32_t *out = bidx + b * bi_bstride + q * budget;
            for (int t = lane; t < budget; t += 64) out[t] = (t < o) ? t : -1;
        }
        return;
    }

    for (int x = tid; x < kIdxQueriesPerWG * kTopkBins; x += 256) (&hist[0][0])[x] = 0;

    bf16x8 afrag[2][8];
    for (int a = 0; a < 2; ++a) {
        const int r = 64 * wave + 32 * a + (lane & 31);
        const int64_t q = q0 + (r >> 2);
        const int h = r & 3;
        for (int s = 0; s < 8; ++s) {
            if (q < L) {
                const bf16_t *src = qrot + b * qrot_bstride + (q * kIdxHeads + h) * kIdxDim + 16 * s + 8 * (lane >> 5);
                afrag[a][s] = *reinterpret_cast<const bf16x8 *>(src);
            } else {
                afrag[a][s] = bf16x8{};
            }
        }
    }
    // The wave scores queries 16*wave + j, j = 8a + 2i + p (p = lane half).
    // Lane j of st_cnt / st_bt / st_ca holds query j's kept count, its
    // threshold bin bt (tau = lower edge of bin bt) and the number of kept
    // scores in bins above bt; tau_v is each lane's copy of its own query's
    // threshold.  Padding queries of a ragged tile get an infinite threshold
    // and keep nothing.
    uint32_t st_cnt = 0, st_ca = 0;
    int st_bt = 0;
    const bool st_live = lane < 16 && q0 + 16 * wave + lane < L;
    float tau_v[2][4];
    uint32_t tn_v[2][4];       // bits of the lower edge of the bin above tau (kept scores at or above it raise st_ca)
    int32_t qo[2][4];
    for (int a = 0; a < 2; ++a)
        for (int i = 0; i < 4; ++i) {
            const int64_t q = q0 + 16 * wave + 8 * a + 2 * i + half;
            qo[a][i] = (q < L) ? static_cast<int32_t>((q_offset + q) >> rsh) : 0;
            tau_v[a][i] = (q < L) ? 0.0f : INFINITY;
            tn_v[a][i] = next_bin_bits(tau_v[a][i]);
        }
    const int64_t o_min = (q_offset + q0) >> rsh;         // causal limit of the tile's first query
    // candidate lists of this workgroup's 64 queries (rows b*L + q0 .. +63); the
    // padding queries of a ragged tile never append (infinite threshold)
    uint2 *__restrict__ wg_cand = cand + (b * L + q0) * cap;
    char *__restrict__ wg_cand_bytes = reinterpret_cast<char *>(wg_cand);   // 32-bit byte offsets below 4 MiB
    // hist indexed by the unclamped bin field: hist_rebased[ql * 128 + (bits >> 20)], bits >> 20 >= base
    uint32_t *hist_rebased = &hist[0][0] - kTopkBinBase;

    const bf16_t *kb = kbar + b * nblk_cap * kIdxDim;
    // k̄ tiles: the next tile is loaded into registers before the current
    // tile's MFMAs and written to LDS after them.
    u32x4 pre[4];
    auto fetch = [&](int64_t cs) {
        for (int it = 0; it < 4; ++it) {
            const int chunk = it * 256 + tid;
            const int64_t blk = cs + (chunk >> 4);
            pre[it] = (blk < nblk_cap) ? *reinterpret_cast<const u32x4 *>(kb + blk * kIdxDim + 8 * (chunk & 15))
                                       : u32x4{0, 0, 0, 0};
        }
    };
    auto put = [&](int buf) {
        for (int it = 0; it < 4; ++it) {
            const int chunk = it * 256 + tid;
            *reinterpret_cast<u32x4 *>(&lds[buf][(chunk >> 4) * kLdsRow + 8 * (chunk & 15)]) = pre[it];
        }
    };

    int buf = 0;
    fetch(0);
    put(0);
    __syncthreads();
    for (int64_t cs = 0; cs < o_hi; cs += kIdxSubCols) {
        const bool more = cs + kIdxSubCols < o_hi;
        if (more) fetch(cs + kIdxSubCols);

        f32x16 acc[2][2];
        for (int ct = 0; ct < 2; ++ct) {
            bf16x8 bfrag[8];
            const bf16_t *brow = &lds[buf][(32 * ct + (lane & 31)) * kLdsRow + 8 * (lane >> 5)];
            for (int s = 0; s < 8; ++s) bfrag[s] = *reinterpret_cast<const bf16x8 *>(brow + 16 * s);
            for (int a = 0; a < 2; ++a) {
                f32x16 c = {};
                for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[a][s], bfrag[s], c, 0, 0, 0);
                acc[a][ct] = c;
            }
        }
        bool any = false;
        // Columns of this tile lie below every query's causal limit except on
        // the last one or two tiles of the row range (queries of a tile span 16
        // blocks), so the causal mask is applied there only.
        auto epilogue = [&](auto masked) {
            for (int a = 0; a < 2; ++a) {
                for (int i = 0; i < 4; ++i) {
                    // lanes 0..31 score query j0, lanes 32..63 query j0 + 1, at
                    // columns cs + 32*ct + lane%32 of the two column tiles
                    const int j0 = 8 * a + 2 * i;
                    uint32_t sb[2];
                    bool keep[2];
                    uint64_t m[2];
                    for (int ct = 0; ct < 2; ++ct) {
                        const int32_t col = static_cast<int32_t>(cs) + 32 * ct + (lane & 31);
                        const f32x16 &c = acc[a][ct];
                        const float s = relu_sum4_fast(c[4 * i], c[4 * i + 1], c[4 * i + 2], c[4 * i + 3]);
                        if constexpr (decltype(masked)::value)
                            keep[ct] = s >= tau_v[a][i] && col < qo[a][i];
                        else
                            keep[ct] = s >= tau_v[a][i];
                        sb[ct] = __float_as_uint(s) & 0x7FFFFFFFu;           // -0 -> +0
                        m[ct] = __builtin_amdgcn_ballot_w64(keep[ct]);
                    }
                    if ((m[0] | m[1]) == 0) continue;                        // wave-uniform
                    any = true;
                    const uint32_t c0 = __builtin_amdgcn_readlane(st_cnt, j0);
                    const uint32_t c1 = __builtin_amdgcn_readlane(st_cnt, j0 + 1);
                    const uint32_t tn = tn_v[a][i];
                    const uint32_t nl0 = static_cast<uint32_t>(__popc(static_cast<uint32_t>(m[0])));
                    const uint32_t nh0 = static_cast<uint32_t>(__popc(static_cast<uint32_t>(m[0] >> 32)));
                    const uint32_t nl1 = static_cast<uint32_t>(__popc(static_cast<uint32_t>(m[1])));
                    const uint32_t nh1 = static_cast<uint32_t>(__popc(static_cast<uint32_t>(m[1] >> 32)));
                    const uint32_t ql = static_cast<uint32_t>(16 * wave + j0 + half);
                    // list positions: the query's kept count, then its column tile 0
                    // entries, then tile 1 (block order); mbcnt counts the whole wave,
                    // so upper-half lanes drop the lower half's count
                    const uint32_t base0 = half ? c1 - nl0 : c0;
                    const uint32_t base1 = half ? c1 + nh0 - nl1 : c0 + nl0;
                    uint64_t am = 0, am1 = 0;
                    for (int ct = 0; ct < 2; ++ct) {
                        const uint64_t a_m = __builtin_amdgcn_ballot_w64(sb[ct] >= tn) & m[ct];
                        if (ct == 0) am = a_m; else am1 = a_m;
                        if (keep[ct]) {
                            const uint32_t below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m[ct] >> 32),
                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m[ct]), 0u));
                            const uint32_t pos = (ct == 0 ? base0 : base1) + below;
                            // a list past its capacity stays in bounds (its row is
                            // recomputed exactly: see the final selection)
                            const uint32_t slot = min(pos, static_cast<uint32_t>(cap) - 1u);
                            const uint32_t col = static_cast<uint32_t>(cs) + 32 * ct + (lane & 31);
                            *reinterpret_cast<uint2 *>(wg_cand_bytes + (ql * static_cast<uint32_t>(cap) + slot) * 8u) =
                                make_uint2(sb[ct], col);
                            // bin = clamp(bits >> 20, base, base + 127) - base, folded into the row address
                            const uint32_t e = min(max(sb[ct] >> 20, static_cast<uint32_t>(kTopkBinBase)),
                                                   static_cast<uint32_t>(kTopkBinBase + kTopkBins - 1));
                            atomicAdd(hist_rebased + ql * kTopkBins + e, 1u);
                        }
                    }
                    const bool l0 = lane == j0, l1 = lane == j0 + 1;
                    st_cnt += l0 ? nl0 + nl1 : (l1 ? nh0 + nh1 : 0u);
                    if (am | am1) {
                        const uint32_t al = static_cast<uint32_t>(__popc(static_cast<uint32_t>(am)) +
                                                                  __popc(static_cast<uint32_t>(am1)));
                        const uint32_t ah = static_cast<uint32_t>(__popc(static_cast<uint32_t>(am >> 32)) +
                                                                  __popc(static_cast<uint32_t>(am1 >> 32)));
                        st_ca += l0 ? al : (l1 ? ah : 0u);
                    }
                }
            }
        };
        if (cs + kIdxSubCols <= o_min)
            epilogue(std::integral_constant<bool, false>{});
        else
            epilogue(std::integral_constant<bool, true>{});
        if (any && __builtin_amdgcn_ballot_w64(st_ca >= static_cast<uint32_t>(budget))) {
            // raise thresholds: while the kept scores above bin bt reach the
            // budget, bin bt + 1's lower edge is a valid threshold
            if (lane < 16) {
                while (st_ca >= static_cast<uint32_t>(budget) && st_bt < kTopkBins - 1) {
                    ++st_bt;
                    st_ca -= hist[16 * wave + lane][st_bt];
                }
            }
            const float st_tau = st_live ? topk_bin_edge(st_bt) : INFINITY;
            for (int a = 0; a < 2; ++a)
                for (int i = 0; i < 4; ++i) {
                    const int j0 = 8 * a + 2 * i;
                    const float ta = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(st_tau), j0));
                    const float tb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(st_tau), j0 + 1));
                    tau_v[a][i] = half ? tb : ta;
                    tn_v[a][i] = next_bin_bits(tau_v[a][i]);
                }
        }
        if (more) put(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
    // ---- final selection of each query, by the wave that owns it.
    __syncthreads();
    // Boundary bin of each query: its final threshold bin bt (the highest bin
    // whose suffix count of kept scores reaches the budget), with st_ca kept
    // scores above it, all selected.
    wave_sync();
    // The k̄ tiles and this wave's histogram rows are now per-wave scratch:
    // boundary keys and the unordered selection in the first, the boundary
    // entries' block ids in the second.
    uint32_t *bkey = reinterpret_cast<uint32_t *>(&lds[0][0]) + wave * (kTopkBMax + kMaxBudget);
    int32_t *sel = reinterpret_cast<int32_t *>(bkey + kTopkBMax);
    int32_t *bid = reinterpret_cast<int32_t *>(&hist[16 * wave][0]);
    for (int j = 0; j < 16; ++j) {
        const int ql = 16 * wave + j;
        const int64_t q = q0 + ql;
        if (q >= L) break;
        const int64_t o = (q_offset + q) >> rsh;
        int32_t *out = bidx + b * bi_bstride + q * budget;
        if (o <= budget) {
            for (int t = lane; t < budget; t += 64) out[t] = (t < o) ? t : -1;
            continue;
        }
        const uint32_t c = __builtin_amdgcn_readlane(st_cnt, j);
        const int bstar = __builtin_amdgcn_readlane(st_bt, j);
        const uint32_t above = __builtin_amdgcn_readlane(st_ca, j);
        const uint32_t k_rem = static_cast<uint32_t>(budget) - above;
        // Inside an interior bin the high score bits are fixed, so (low 20
        // score bits, boundary ordinal) packs (score desc, block desc) into one
        // 32-bit key.  The two clamped end bins keep full score bits.
        const bool clamped = bstar == 0 || bstar == kTopkBins - 1;
        bool fail = c > static_cast<uint32_t>(cap) || bstar < 0;
        uint32_t nb = 0, ng = 0;
        if (!fail) {
            // one pass over the list, kU entries per lane in flight: the
            // higher-bin blocks go to sel[], the boundary-bin ones to bkey/bid
            const uint2 *lst = wg_cand + ql * cap;
            for (uint32_t p0 = 0; p0 < c; p0 += 64 * kU) {
                uint2 e[kU];
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const uint32_t p = p0 + 64 * u + lane;
                    e[u] = (p < c) ? lst[p] : make_uint2(0xFFFFFFFFu, 0u);
                }
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const bool valid = e[u].x != 0xFFFFFFFFu;
                    const int bn = topk_bin(__uint_as_float(e[u].x));
                    const bool g = valid && bn > bstar;
                    const bool eq = valid && bn == bstar;
                    const uint64_t gm = __builtin_amdgcn_ballot_w64(g);
                    const uint64_t em = __builtin_amdgcn_ballot_w64(eq);
                    if (g) {
                        const uint32_t t = ng + lanes_below(gm);
                        if (t < static_cast<uint32_t>(kMaxBudget)) sel[t] = static_cast<int32_t>(e[u].y);
                    }
                    if (eq) {
                        const uint32_t t = nb + lanes_below(em);
                        if (t < static_cast<uint32_t>(kTopkBMax)) {
                            bkey[t] = clamped ? e[u].x : ((e[u].x & 0xFFFFFu) << 11) | t;
                            bid[t] = static_cast<int32_t>(e[u].y);
                        }
                    }
                    ng += static_cast<uint32_t>(__popcll(gm));
                    nb += static_cast<uint32_t>(__popcll(em));
                }
            }
            fail = ng != above || nb < k_rem || nb > static_cast<uint32_t>(kTopkBMax) ||
                   (clamped && nb != k_rem && nb > static_cast<uint32_t>(kTopkRankMax));
        }
        if (fail) {                                   // exact recompute by select_fixup_kernel
            if (lane == 0) {
                const int slot = atomicAdd(&ovf[0], 1);
                ovf[1 + slot] = static_cast<int32_t>(b * L + q);
            }
            continue;
        }
        wave_sync();
        // the k_rem best boundary entries join sel[above ..), in list order
        // except on the clamped path (rank order)
        bool in_order = true;
        if (nb == k_rem) {
            for (uint32_t t = lane; t < nb; t += 64) sel[above + t] = bid[t];
        } else if (clamped) {
            in_order = false;
            // rank = entries ahead in (score desc, ordinal desc); ranks are unique
            for (uint32_t t = lane; t < nb; t += 64) {
                const uint32_t kx = bkey[t];
                uint32_t r = 0;
                for (uint32_t u = 0; u < nb; ++u) {
                    const uint32_t ky = bkey[u];
                    r += (ky > kx) || (ky == kx && u > t);
                }
                if (r < k_rem) sel[above + r] = bid[t];
            }
        } else {
            const uint32_t n64 = (nb + 63) >> 6;
            if (n64 <= 1)       boundary_mark<1>(bkey, nb, k_rem, lane);
            else if (n64 <= 2)  boundary_mark<2>(bkey, nb, k_rem, lane);
            else if (n64 <= 4)  boundary_mark<4>(bkey, nb, k_rem, lane);
            else if (n64 <= 8)  boundary_mark<8>(bkey, nb, k_rem, lane);
            else if (n64 <= 16) boundary_mark<16>(bkey, nb, k_rem, lane);
            else                boundary_mark<32>(bkey, nb, k_rem, lane);
            wave_sync();
            // the marked entries, compacted in list order
            uint32_t pos = static_cast<uint32_t>(above);
            for (uint32_t t0 = 0; t0 < nb; t0 += 64) {
                const uint32_t t = t0 + lane;
                const bool f = t < nb && bkey[t] != 0u;
                const uint64_t fm = __builtin_amdgcn_ballot_w64(f);
                if (f) sel[pos + lanes_below(fm)] = bid[t];
                pos += static_cast<uint32_t>(__popcll(fm));
            }
        }
        wave_sync();
        // ascending block order
        if (in_order) {
            if (budget <= 64)       emit_merged<1>(sel, static_cast<int>(above), budget, out, lane);
            else if (budget <= 128) emit_merged<2>(sel, static_cast<int>(above), budget, out, lane);
            else if (budget <= 256) emit_merged<4>(sel, static_cast<int>(above), budget, out, lane);
            else                    emit_merged<8>(sel, static_cast<int>(above), budget, out, lane);
        } else {
            if (budget <= 64)       emit_sorted<1>(sel, budget, out, lane);
            else if (budget <= 128) emit_sorted<2>(sel, budget, out, lane);
            else if (budget <= 256) emit_sorted<4>(sel, budget, out, lane);
            else                    emit_sorted<8>(sel, budget, out, lane);
        }
        wave_sync();
    }
}

hipError_t launch_indexer_topk(hipStream_t st, int32_t B, int64_t L, int64_t q_offset, int rsh, int64_t nblk_cap,
                               int budget, int cap, const bf16_t *qrot, int64_t qrot_bstride, const bf16_t *kbar,
                               uint2 *cand, int32_t *bidx, int64_t bi_bstride, int32_t *ovf)
{
    if (L <= 0) return hipSuccess;
    dim3 grid(static_cast<unsigned>((L + kIdxQueriesPerWG - 1) / kIdxQueriesPerWG), static_cast<unsigned>(B));
    hipLaunchKernelGGL(indexer_topk_kernel, grid, dim3(256), 0, st, L, q_offset, rsh, nblk_cap, budget, cap, qrot,
                       qrot_bstride, kbar, cand, bidx, bi_bstride, ovf);
    return hipGetLastError();
}

// Clear n words (counters that a later kernel accumulates into).
__global__ void zero_words_kernel(int32_t *p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

hipError_t launch_zero_words(hipStream_t st, int32_t *p, int64_t n) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_words_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

}  // namespace qsa
