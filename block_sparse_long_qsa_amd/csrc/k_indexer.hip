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
// 0 .. floor(p_last/4) in k̄ tiles of 64, computing the same MFMA scores as
// indexer_scores_kernel.  Each query keeps
//   * a running threshold tau (fp32), below which a block can no longer be in
//     its top `budget`: tau is the lower edge of the highest bin of a 128-bin
//     log histogram (8 bins per octave over [2^-8, 2^8)) of the scores kept so
//     far whose suffix count reaches `budget` -- at least `budget` kept scores
//     are >= tau, so the budget-th largest score is >= tau;
//   * the list of (score, block) pairs with score >= tau, appended in ascending
//     block order (ballot + prefix count per 32-column tile).
// Queries are owned by one wave each, so the histograms, counters and
// thresholds need no workgroup barrier.  The exact top-`budget` is then taken
// from the short list by select_compact_kernel.  A list that would outgrow
// `cap` keeps counting without storing; its row is recomputed exactly there.
// Workgroups are issued latest-queries-first (longest rows first).
constexpr int kTopkBins = 128;
constexpr int kTopkBinBase = 951;      // bin 1 = [2^-8, 2^-8 * 1.125); 952 = (127 - 8) * 8
constexpr uint32_t kTauRefresh = 32;    // appends between threshold refreshes

__device__ __forceinline__ int topk_bin(float s) {
    const int b = static_cast<int>(__float_as_uint(s) >> 20) - kTopkBinBase;
    return b < 0 ? 0 : (b >= kTopkBins ? kTopkBins - 1 : b);
}
__device__ __forceinline__ float topk_bin_edge(int b) {
    return b <= 0 ? 0.0f : __uint_as_float(static_cast<uint32_t>(b + kTopkBinBase) << 20);
}

__global__ __launch_bounds__(256, 2) void indexer_topk_kernel(
    int64_t L, int64_t q_offset, int64_t nblk_cap, int budget, int cap,
    const bf16_t *__restrict__ qrot, int64_t qrot_bstride, const bf16_t *__restrict__ kbar,
    float *__restrict__ cand_score, int32_t *__restrict__ cand_idx, int32_t *__restrict__ cand_count,
    int32_t *__restrict__ cand_meta)
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
    const int64_t o_hi = (q_offset + q_last) / kBlock;
    if (o_hi <= budget) return;                 // every row of the tile keeps all its candidates

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
    // Their kept counts, appends since the last threshold refresh and
    // thresholds live in lane j of st_cnt / st_since / st_tau; tau_v is each
    // lane's copy of its own query's threshold.  Padding queries of a ragged
    // tile get an infinite threshold and keep nothing.
    uint32_t st_cnt = 0, st_since = 0;
    float st_tau = (lane < 16 && q0 + 16 * wave + lane < L) ? 0.0f : INFINITY;
    float tau_v[2][4];
    int32_t qo[2][4];
    for (int a = 0; a < 2; ++a)
        for (int i = 0; i < 4; ++i) {
            const int64_t q = q0 + 16 * wave + 8 * a + 2 * i + half;
            qo[a][i] = (q < L) ? static_cast<int32_t>((q_offset + q) / kBlock) : 0;
            tau_v[a][i] = (q < L) ? 0.0f : INFINITY;
        }
    const int64_t o_min = (q_offset + q0) / kBlock;         // causal limit of the tile's first query
    // candidate lists of this workgroup's 64 queries (rows b*L + q0 .. +63); the
    // padding queries of a ragged tile never append (infinite threshold)
    float *__restrict__ wg_score = cand_score + (b * L + q0) * cap;
    int32_t *__restrict__ wg_idx = cand_idx + (b * L + q0) * cap;

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
                    for (int ct = 0; ct < 2; ++ct) {
                        const int32_t col = static_cast<int32_t>(cs) + 32 * ct + (lane & 31);
                        const f32x16 &c = acc[a][ct];
                        const float s = relu_sum4_fast(c[4 * i], c[4 * i + 1], c[4 * i + 2], c[4 * i + 3]);
                        bool keep;
                        if constexpr (decltype(masked)::value)
                            keep = s >= tau_v[a][i] && col < qo[a][i];
                        else
                            keep = s >= tau_v[a][i];
                        const uint64_t m = __builtin_amdgcn_ballot_w64(keep);
                        if (m == 0) continue;                            // wave-uniform
                        any = true;
                        const int j0 = 8 * a + 2 * i;                    // queries j0 (lanes 0..31), j0 + 1
                        const uint32_t m0 = static_cast<uint32_t>(m), m1 = static_cast<uint32_t>(m >> 32);
                        const uint32_t n0 = static_cast<uint32_t>(__popc(m0)), n1 = static_cast<uint32_t>(__popc(m1));
                        if (keep) {
                            // position = kept count of the lane's query + kept lanes below it in its half
                            const uint32_t b0 = __builtin_amdgcn_readlane(st_cnt, j0);
                            const uint32_t b1 = __builtin_amdgcn_readlane(st_cnt, j0 + 1) - n0;
                            const uint32_t below = __builtin_amdgcn_mbcnt_hi(m1, __builtin_amdgcn_mbcnt_lo(m0, 0u));
                            const uint32_t pos = (half ? b1 : b0) + below;
                            const uint32_t ql = static_cast<uint32_t>(16 * wave + j0 + half);
                            const float sc = __uint_as_float(__float_as_uint(s) & 0x7FFFFFFFu);   // -0 -> +0
                            if (pos < static_cast<uint32_t>(cap)) {
                                const uint32_t off = ql * static_cast<uint32_t>(cap) + pos;
                                wg_score[off] = sc;
                                wg_idx[off] = col;
                            }
                            atomicAdd(&hist[ql][topk_bin(sc)], 1u);
                        }
                        const uint32_t add = (lane == j0) ? n0 : (lane == j0 + 1 ? n1 : 0u);
                        st_cnt += add;
                        st_since += add;
                    }
                }
            }
        };
        if (cs + kIdxSubCols <= o_min)
            epilogue(std::integral_constant<bool, false>{});
        else
            epilogue(std::integral_constant<bool, true>{});
        if (any) {
            // refresh the thresholds of queries that kept enough new scores: the
            // highest bin whose suffix count reaches the budget gives tau
            uint64_t todo = __builtin_amdgcn_ballot_w64(lane < 16 && st_since >= kTauRefresh);
            if (todo) {
                while (todo) {
                    const int j = __builtin_ctzll(todo);
                    todo &= todo - 1;
                    const int ql = 16 * wave + j;
                    const uint32_t h0 = hist[ql][2 * lane], h1 = hist[ql][2 * lane + 1];
                    uint32_t incl = h0 + h1;                           // kept scores in bins >= 2*lane
                    for (int off = 1; off < 64; off <<= 1) {
                        const uint32_t other = __shfl_down(incl, off);
                        if (lane + off < 64) incl += other;
                    }
                    const uint32_t c1 = incl - h0;                     // bins >= 2*lane + 1
                    const int cand = (c1 >= static_cast<uint32_t>(budget)) ? 2 * lane + 1
                                     : (incl >= static_cast<uint32_t>(budget) ? 2 * lane : -1);
                    const uint64_t vm = __builtin_amdgcn_ballot_w64(cand >= 0);
                    if (vm != 0) {
                        const int hi = 63 - __clzll(vm);
                        const float t = topk_bin_edge(__shfl(cand, hi));
                        if (lane == j && t > st_tau) st_tau = t;
                    }
                    if (lane == j) st_since = 0;
                }
                for (int a = 0; a < 2; ++a)
                    for (int i = 0; i < 4; ++i) tau_v[a][i] = __shfl(st_tau, 8 * a + 2 * i + half);
            }
        }
        if (more) put(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
    // final boundary bin of each query: the highest bin whose suffix count
    // reaches the budget, and the number of kept scores above it
    for (int j = 0; j < 16; ++j) {
        const int ql = 16 * wave + j;
        const int64_t q = q0 + ql;
        if (q >= L) break;
        const uint32_t h0 = hist[ql][2 * lane], h1 = hist[ql][2 * lane + 1];
        uint32_t incl = h0 + h1;
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t other = __shfl_down(incl, off);
            if (lane + off < 64) incl += other;
        }
        const uint32_t c1 = incl - h0;
        const int cand = (c1 >= static_cast<uint32_t>(budget)) ? 2 * lane + 1
                         : (incl >= static_cast<uint32_t>(budget) ? 2 * lane : -1);
        const uint32_t above = (cand == 2 * lane + 1) ? c1 - h1 : incl - h0;    // bins > cand
        const uint64_t vm = __builtin_amdgcn_ballot_w64(cand >= 0);
        const int hi = vm ? 63 - __clzll(vm) : 0;
        const int bin = vm ? __shfl(cand, hi) : -1;
        const uint32_t ab = __shfl(above, hi);
        const uint32_t n = __shfl(st_cnt, j);
        if (lane == 0) {
            cand_count[b * L + q] = static_cast<int32_t>(n);
            cand_meta[2 * (b * L + q)] = bin;
            cand_meta[2 * (b * L + q) + 1] = static_cast<int32_t>(vm ? ab : 0);
        }
    }
}

hipError_t launch_indexer_topk(hipStream_t st, int32_t B, int64_t L, int64_t q_offset, int64_t nblk_cap, int budget,
                               int cap, const bf16_t *qrot, int64_t qrot_bstride, const bf16_t *kbar,
                               float *cand_score, int32_t *cand_idx, int32_t *cand_count, int32_t *cand_meta)
{
    if (L <= 0) return hipSuccess;
    dim3 grid(static_cast<unsigned>((L + kIdxQueriesPerWG - 1) / kIdxQueriesPerWG), static_cast<unsigned>(B));
    hipLaunchKernelGGL(indexer_topk_kernel, grid, dim3(256), 0, st, L, q_offset, nblk_cap, budget, cap, qrot,
                       qrot_bstride, kbar, cand_score, cand_idx, cand_count, cand_meta);
    return hipGetLastError();
}

}  // namespace qsa
