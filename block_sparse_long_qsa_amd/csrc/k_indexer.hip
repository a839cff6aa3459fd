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
#include "qsa_common.h"

namespace qsa {

constexpr int kIdxQueriesPerWG = 64;
constexpr int kIdxColsPerWG = 512;
constexpr int kIdxSubCols = 64;
constexpr int kLdsRow = kIdxDim + 8;   // padded row (elements) against bank conflicts

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

}  // namespace qsa
