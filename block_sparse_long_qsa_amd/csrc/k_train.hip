// Indexer loss of the training path (PyTorchKR post "Qwen3.8-Flash-Next, 1/9의
// 학습 비용으로 …", section "QSA: 인덱서 자체의 비용을 줄이는 희소 어텐션": the
// indexer learns the attention distribution matched per micro-block with max
// pooling, and a fused kernel computes the sparse attention output and the
// indexer's KL-divergence loss without materialising intermediates).
//
// For query p with selected blocks S(p) (the valid entries of its selection):
//   teacher  A_b = max over the block's 4 tokens of the head-mean attention
//            probability (softmax over the token set T(p), from the log-sum-exp
//            attend_stats_kernel stored), pi_b = A_b / Z, Z = sum A;
//   student  s_b = softmax over S(p) of I_b = sum_h ReLU(<q~_h, k̄_b>);
//   loss     KL(pi || s) = (sum A ln A) / Z - ln Z - (sum A I) / Z + lse(I).
// Backward (the teacher is a constant): g_b = dkl (s_b - pi_b);
//   dq~_h += g_b [<q~_h, k̄_b> > 0] k̄_b  and  dk̄_b += g_b sum_h [..] q~_h
//   (atomics), then the transposed rotations and the pooling's 1/4.
//
// One workgroup of two waves per query.  Wave w recomputes the logits of KV
// group w over the selected blocks, 8 per chunk with the attention kernel's
// MFMA layout, and sums its 12 heads' probabilities per token (xor shuffles
// inside each 16-lane row); the two groups' sums meet in LDS.  Wave 0 scores
// the chunk's 8 blocks with one 16x16x32 MFMA tile (rows = the 4 indexer
// heads, columns = blocks) and keeps the running sums; in the backward wave 0
// accumulates dq~ and wave 1 adds the dk̄ contributions.  LDS is double
// buffered by chunk parity, so one barrier per chunk separates writers and
// readers (two in the backward).
#include "qsa_common.h"
#include "attend_parts.h"

namespace qsa {

template <bool BWD>
__global__ __launch_bounds__(128) void train_kl_kernel(
    Tables tab, int64_t L, int64_t nblk_cap, int budget, float c2,
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k_cache, const bf16_t *__restrict__ kbar,
    const bf16_t *__restrict__ qrot, const int32_t *__restrict__ block_idx, float *__restrict__ stats,
    float *__restrict__ kl, const float *__restrict__ dkl, float *__restrict__ dq_idx, float *__restrict__ dkbar)
{
    __shared__ float hs[2][2][2][16];      // [buffer][group][tile][4 * entry-in-tile + token]
    __shared__ float cf[2][kIdxHeads][8];  // [buffer][head][entry]: g_b [logit > 0]
    __shared__ int32_t ids[2][8];          // [buffer][entry]: block id, -1 if not a valid selected block
    const int lane = threadIdx.x & 63;
    const int grp = threadIdx.x >> 6;
    const int64_t i = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t row = b * L + i;
    const int64_t pos = i;
    const int64_t o = pos / kBlock;
    const int n_sel = static_cast<int>(o < budget ? o : budget);
    const int h = lane & 15, g = lane >> 4;
    float *st = stats + row * kTrainStats;

    bf16x8 qf[8];
    load_q_frags(q + row * kQHeads * kHeadDim, grp, pos, tab, qf);
    const float lse2 = (h < kGroup) ? st[grp * kGroup + h] * kLog2e : 0.f;
    const bf16_t *kc = k_cache + kcache_block_base(b, grp, 0, nblk_cap);
    const bf16_t *kb = kbar + b * nblk_cap * kIdxDim;
    const int32_t *sel = block_idx + row * budget;
    const bf16_t *qi = qrot + row * kIdxHeads * kIdxDim;

    bf16x8 af[4];                          // wave 0: indexer query, MFMA A rows = heads 0..3
    for (int s = 0; s < 4; ++s)
        af[s] = (grp == 0 && h < kIdxHeads) ? *reinterpret_cast<const bf16x8 *>(qi + h * kIdxDim + 32 * s + 8 * g)
                                            : bf16x8{};
    // forward running sums (wave 0, lane e < 8 holds chunk entry e)
    float zA = 0.f, uA = 0.f, wA = 0.f, im = -INFINITY, ie = 0.f;
    int nval = 0;
    // backward state
    float Z = 1.f, lse_i = 0.f, gscale = 0.f;
    if (BWD) {
        Z = expf(st[kTrainStats - 8]);
        lse_i = st[kTrainStats - 7];
        gscale = dkl[row];
    }
    float dq[8];                           // wave 0: head lane/16, dims 8*(lane%16) .. +7
    float qk[2][kIdxHeads];                // wave 1: dims 2*lane, 2*lane+1 of the 4 heads of q~
    for (int k = 0; k < 8; ++k) dq[k] = 0.f;
    for (int k = 0; k < 2; ++k)
        for (int hh = 0; hh < kIdxHeads; ++hh)
            qk[k][hh] = (BWD && grp == 1) ? bf16_to_f32(qi[hh * kIdxDim + 2 * lane + k]) : 0.f;

    const int nch = (n_sel + kChunkBlocks - 1) / kChunkBlocks;
    for (int c = 0; c < nch; ++c) {
        const int buf = c & 1;
        const int lb = kChunkBlocks * c;
        // ---- K~ tiles (token row h of tile t: entry lb + 4t + h/4, token h%4)
        bf16x8 kf[2][8];
        bool oval[2];
        for (int t = 0; t < 2; ++t) {
            const int li = lb + 4 * t + (h >> 2);
            const int64_t id = sel[li < n_sel ? li : 0];
            const bool ok = li < n_sel && id >= 0 && id < o;
            const bf16_t *src = kc + (ok ? id : 0) * kBlockElems + (h & 3) * 32 + 8 * g;
            for (int s = 0; s < 8; ++s) kf[t][s] = *reinterpret_cast<const bf16x8 *>(src + s * 128);
            const int lo = lb + 4 * t + g;                        // entry of this lane's outputs
            const int64_t ido = sel[lo < n_sel ? lo : 0];
            oval[t] = lo < n_sel && ido >= 0 && ido < o;
        }
        // ---- S^T = K~ Q~^T; lane holds tokens 0..3 of entry lb + 4t + g for head h
        for (int t = 0; t < 2; ++t) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t][s], qf[s], acc, 0, 0, 0);
            for (int j = 0; j < 4; ++j) {
                float pj = (oval[t] && h < kGroup) ? exp2f(acc[j] * c2 - lse2) : 0.f;
                pj += __shfl_xor(pj, 1);
                pj += __shfl_xor(pj, 2);
                pj += __shfl_xor(pj, 4);
                pj += __shfl_xor(pj, 8);
                if (h == 0) hs[buf][grp][t][4 * g + j] = pj;
            }
        }
        __syncthreads();
        if (grp == 0) {
            // ---- student scores: MFMA B column h = chunk entry h (0..7 used)
            const int le = lb + h;
            const int64_t id = sel[(h < kChunkBlocks && le < n_sel) ? le : 0];
            const bool ev = h < kChunkBlocks && le < n_sel && id >= 0 && id < o;
            const bf16_t *ksrc = kb + (ev ? id : 0) * kIdxDim + 8 * g;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < 4; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s], *reinterpret_cast<const bf16x8 *>(ksrc + 32 * s),
                                                              acc, 0, 0, 0);
            if (lane < kChunkBlocks) {         // g == 0: heads 0..3 against entry `lane`
                const float I = fmaxf(acc[0], 0.f) + fmaxf(acc[1], 0.f) + fmaxf(acc[2], 0.f) + fmaxf(acc[3], 0.f);
                const int t = lane >> 2, ge = lane & 3;
                float A = 0.f;
                for (int j = 0; j < 4; ++j) A = fmaxf(A, hs[buf][0][t][4 * ge + j] + hs[buf][1][t][4 * ge + j]);
                A *= 1.0f / kQHeads;
                if (!BWD) {
                    if (ev) {
                        zA += A;
                        uA += (A > 0.f) ? A * logf(A) : 0.f;
                        wA += A * I;
                        if (I > im) {
                            ie = ie * expf(im - I) + 1.f;
                            im = I;
                        } else {
                            ie += expf(I - im);
                        }
                        ++nval;
                    }
                } else {
                    const float gc = ev ? gscale * (expf(I - lse_i) - A / Z) : 0.f;
                    for (int hh = 0; hh < kIdxHeads; ++hh) cf[buf][hh][lane] = (acc[hh] > 0.f) ? gc : 0.f;
                    ids[buf][lane] = ev ? static_cast<int32_t>(id) : -1;
                }
            }
        }
        if (BWD) {
            __syncthreads();
            if (grp == 0) {
                const int hh = lane >> 4, d0 = 8 * (lane & 15);
                for (int e = 0; e < kChunkBlocks; ++e) {
                    const int32_t id = ids[buf][e];
                    const float cv = cf[buf][hh][e];
                    if (id < 0 || cv == 0.f) continue;
                    const u32x4 kv = *reinterpret_cast<const u32x4 *>(kb + static_cast<int64_t>(id) * kIdxDim + d0);
                    for (int k = 0; k < 4; ++k) {
                        dq[2 * k] += cv * __uint_as_float(kv[k] << 16);
                        dq[2 * k + 1] += cv * __uint_as_float(kv[k] & 0xFFFF0000u);
                    }
                }
            } else {
                for (int e = 0; e < kChunkBlocks; ++e) {
                    const int32_t id = ids[buf][e];
                    if (id < 0) continue;
                    float v0 = 0.f, v1 = 0.f;
                    for (int hh = 0; hh < kIdxHeads; ++hh) {
                        v0 += cf[buf][hh][e] * qk[0][hh];
                        v1 += cf[buf][hh][e] * qk[1][hh];
                    }
                    float *dst = dkbar + (b * nblk_cap + id) * kIdxDim + 2 * lane;
                    if (v0 != 0.f) atomicAdd(dst, v0);
                    if (v1 != 0.f) atomicAdd(dst + 1, v1);
                }
            }
        }
    }

    if (grp != 0) return;
    if (!BWD) {
        for (int off = 1; off < 64; off <<= 1) {
            zA += __shfl_xor(zA, off);
            uA += __shfl_xor(uA, off);
            wA += __shfl_xor(wA, off);
            nval += __shfl_xor(nval, off);
        }
        float M = im;
        for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
        float E = (nval > 0 && ie > 0.f) ? ie * expf(im - M) : 0.f;
        for (int off = 1; off < 64; off <<= 1) E += __shfl_xor(E, off);
        if (lane == 0) {
            const float lnz = nval > 0 ? logf(zA) : 0.f;
            const float lsei = nval > 0 ? M + logf(E) : 0.f;
            kl[row] = nval > 1 ? uA / zA - lnz - wA / zA + lsei : 0.f;
            st[kTrainStats - 8] = lnz;
            st[kTrainStats - 7] = lsei;
            for (int k = kTrainStats - 6; k < kTrainStats; ++k) st[k] = 0.f;
        }
        return;
    }
    // dq_idx = transposed rotation of dq~ at pos: pairs (j, j + 32) sit in lanes
    // c and c + 4 of the head's 16-lane row, c = lane % 16 < 4
    float pv[8];
    for (int k = 0; k < 8; ++k) pv[k] = __shfl_xor(dq[k], 4);
    const int cl = lane & 15;
    const int hh = lane >> 4;
    float outv[8];
    if (cl < 8) {
        const float *cs = tab.cos + pos * kPairs + 8 * (cl & 3);
        const float *sn = tab.sin + pos * kPairs + 8 * (cl & 3);
        for (int k = 0; k < 8; ++k)
            outv[k] = (cl < 4) ? dq[k] * cs[k] + pv[k] * sn[k] : dq[k] * cs[k] - pv[k] * sn[k];
    } else {
        for (int k = 0; k < 8; ++k) outv[k] = dq[k];
    }
    float *dst = dq_idx + (row * kIdxHeads + hh) * kIdxDim + 8 * cl;
    *reinterpret_cast<f32x4 *>(dst) = f32x4{outv[0], outv[1], outv[2], outv[3]};
    *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{outv[4], outv[5], outv[6], outv[7]};
}

// dk_idx[b][t] = 1/4 (transposed rotation at 4*blk of dk̄[b][blk]), blk = t/4,
// for tokens of complete blocks; 0 for the tokens of a trailing partial block
// (never scored).  One thread per (token, dim).
__global__ __launch_bounds__(256) void dk_idx_kernel(Tables tab, int32_t B, int64_t L, int64_t nblk_cap,
                                                     const float *__restrict__ dkbar, float *__restrict__ dk_idx)
{
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (gid >= static_cast<int64_t>(B) * L * kIdxDim) return;
    const int d = static_cast<int>(gid % kIdxDim);
    const int64_t rowt = gid / kIdxDim;
    const int64_t b = rowt / L;
    const int64_t t = rowt - b * L;
    const int64_t blk = t / kBlock;
    float v = 0.f;
    if (kBlock * blk + kBlock - 1 < L) {
        const float *src = dkbar + (b * nblk_cap + blk) * kIdxDim;
        const float *cs = tab.cos + kBlock * blk * kPairs;
        const float *sn = tab.sin + kBlock * blk * kPairs;
        if (d < kPairs)
            v = src[d] * cs[d] + src[d + kPairs] * sn[d];
        else if (d < 2 * kPairs)
            v = src[d] * cs[d - kPairs] - src[d - kPairs] * sn[d - kPairs];
        else
            v = src[d];
        v *= 0.25f;
    }
    dk_idx[gid] = v;
}

hipError_t launch_train_kl(const Tables &tab, hipStream_t st, bool backward, int32_t B, int64_t L, int64_t nblk_cap,
                           int budget, float sigma, const bf16_t *q, const bf16_t *k_cache, const bf16_t *kbar,
                           const bf16_t *qrot, const int32_t *block_idx, float *stats, float *kl, const float *dkl,
                           float *dq_idx, float *dkbar)
{
    if (L <= 0) return hipSuccess;
    dim3 grid(static_cast<unsigned>(L), static_cast<unsigned>(B));
    if (backward)
        hipLaunchKernelGGL(train_kl_kernel<true>, grid, dim3(128), 0, st, tab, L, nblk_cap, budget, sigma * kLog2e, q,
                           k_cache, kbar, qrot, block_idx, stats, kl, dkl, dq_idx, dkbar);
    else
        hipLaunchKernelGGL(train_kl_kernel<false>, grid, dim3(128), 0, st, tab, L, nblk_cap, budget, sigma * kLog2e,
                           q, k_cache, kbar, qrot, block_idx, stats, kl, dkl, dq_idx, dkbar);
    return hipGetLastError();
}

hipError_t launch_dk_idx(const Tables &tab, hipStream_t st, int32_t B, int64_t L, int64_t nblk_cap, const float *dkbar,
                         float *dk_idx)
{
    const int64_t total = static_cast<int64_t>(B) * L * kIdxDim;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(dk_idx_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, st, tab, B, L,
                       nblk_cap, dkbar, dk_idx);
    return hipGetLastError();
}

}  // namespace qsa
