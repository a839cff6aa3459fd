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
    Tables tab, int64_t L, int64_t row0, int64_t nblk_cap, int budget, float c2,
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k_cache, const bf16_t *__restrict__ kbar,
    const bf16_t *__restrict__ qrot, const int32_t *__restrict__ block_idx, float *__restrict__ stats,
    float *__restrict__ kl, const float *__restrict__ dkl, float *__restrict__ dq_idx, float *__restrict__ dkbar)
{
    __shared__ float hs[2][2][2][16];      // [buffer][group][tile][4 * entry-in-tile + token]
    __shared__ float cf[2][kIdxHeads][8];  // [buffer][head][entry]: g_b [logit > 0]
    __shared__ int32_t ids[2][8];          // [buffer][entry]: block id, -1 if not a valid selected block
    const int lane = threadIdx.x & 63;
    const int grp = threadIdx.x >> 6;
    const int64_t i = row0 + blockIdx.x;       // launches cover rows row0 .. of L
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

// ---------------------------------------------------------------------------
// Backward of the sparse attention (the backbone's gradient): for query p and
// KV group g over its token set T(p), with P = exp(sigma S - lse) and
// D_h = <dO_h, O_h>:
//   dS = P (dO V^T - D),  dQ~ = sigma dS K~,  dK~ += sigma dS^T Q~,  dV += P^T dO,
// then dq = R(p)^T dQ~ and dk = R(t)^T dK~ (dims 0..63).  One wave per (group,
// query) walks the query's chunks like the forward; the contractions over
// tokens and heads read operands that LDS holds in the layout each MFMA wants:
// Q~^T and dO^T [dim][head] (once per query), P^T and dS^T [token][head], dS
// [head][token] and the chunk's K~ [token][dim].  V enters token-major for
// dP^T = V dO^T: each lane loads the 64 bytes holding 8 dims x 4 tokens of its
// block and keeps its token's 8 values.  dQ~ stays in registers; dK~ and dV
// are added to the fp32 outputs with atomics (a token is attended by many
// queries).  Masked tokens (invalid entries, the own block past p) take part
// as exact zeros: their cache slots may hold any bits.
__global__ __launch_bounds__(64) void attend_backward_kernel(
    Tables tab, int64_t L, int64_t row0, int64_t nblk_cap, int budget, float c2, float sigma,
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k_cache, const bf16_t *__restrict__ v_cache,
    const int32_t *__restrict__ block_idx, const bf16_t *__restrict__ out, const bf16_t *__restrict__ dout,
    const float *__restrict__ stats, float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dv)
{
    __shared__ __attribute__((aligned(16))) bf16_t qT[kHeadDim][16];
    __shared__ __attribute__((aligned(16))) bf16_t oT[kHeadDim][16];
    __shared__ __attribute__((aligned(16))) bf16_t pT[32][16];
    __shared__ __attribute__((aligned(16))) bf16_t sT[32][16];
    __shared__ __attribute__((aligned(16))) bf16_t sH[16][32];
    __shared__ __attribute__((aligned(16))) bf16_t kt[32][kHeadDim];
    const int lane = threadIdx.x;
    const int64_t i = row0 + blockIdx.x;
    const int grp = blockIdx.y;      // group-major within a launch: each group's queries run together
    const int64_t b = blockIdx.z;
    const int64_t row = b * L + i;
    const int64_t pos = i;
    const int64_t o = pos / kBlock;
    const int own_last = static_cast<int>(pos - o * kBlock);
    const int n_sel = static_cast<int>(o < budget ? o : budget);
    const int nchunks = list_chunks(n_sel, o, o);
    const int h = lane & 15, g = lane >> 4;

    bf16x8 qf[8], dof[8];
    load_q_frags(q + row * kQHeads * kHeadDim, grp, pos, tab, qf);
    const bf16_t *dorow = dout + (row * kQHeads + grp * kGroup + h) * kHeadDim;
    const bf16_t *orow = out + (row * kQHeads + grp * kGroup + h) * kHeadDim;
    float dsum = 0.f;
    for (int s = 0; s < 8; ++s) {
        if (h < kGroup) {
            const u32x4 dw = *reinterpret_cast<const u32x4 *>(dorow + 32 * s + 8 * g);
            const u32x4 ow = *reinterpret_cast<const u32x4 *>(orow + 32 * s + 8 * g);
            dof[s] = __builtin_bit_cast(bf16x8, dw);
            for (int m = 0; m < 4; ++m)
                dsum += __uint_as_float(dw[m] << 16) * __uint_as_float(ow[m] << 16) +
                        __uint_as_float(dw[m] & 0xFFFF0000u) * __uint_as_float(ow[m] & 0xFFFF0000u);
        } else {
            dof[s] = bf16x8{};
        }
    }
    dsum += __shfl_xor(dsum, 16);
    dsum += __shfl_xor(dsum, 32);
    const float Dh = dsum;
    const float lse2 = (h < kGroup) ? stats[row * kTrainStats + grp * kGroup + h] * kLog2e : 0.f;
    // Q~^T and dO^T in LDS: lane (h, g) holds dims 32s + 8g + e of head h
    for (int s = 0; s < 8; ++s) {
        const u32x4 qw = __builtin_bit_cast(u32x4, qf[s]);
        const u32x4 dw = __builtin_bit_cast(u32x4, dof[s]);
        for (int m = 0; m < 4; ++m) {
            const int d = 32 * s + 8 * g + 2 * m;
            qT[d][h] = static_cast<bf16_t>(qw[m] & 0xFFFFu);
            qT[d + 1][h] = static_cast<bf16_t>(qw[m] >> 16);
            oT[d][h] = static_cast<bf16_t>(dw[m] & 0xFFFFu);
            oT[d + 1][h] = static_cast<bf16_t>(dw[m] >> 16);
        }
    }
    f32x4 dqa[16];
    for (int n = 0; n < 16; ++n) dqa[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16_t *kc = k_cache + kcache_block_base(b, grp, 0, nblk_cap);
    const bf16_t *vc = v_cache + kcache_block_base(b, grp, 0, nblk_cap);
    const int32_t *sel = block_idx + row * budget;
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        const int lb = kChunkBlocks * c;
        int64_t kblk[2], oblk[2];
        uint32_t kmask[2], omask[2];
        for (int t = 0; t < 2; ++t) list_entry(sel, 0, n_sel, o, o, lb + 4 * t + (h >> 2), own_last, kblk[t], kmask[t]);
        for (int t = 0; t < 2; ++t) list_entry(sel, 0, n_sel, o, o, lb + 4 * t + g, own_last, oblk[t], omask[t]);
        const int tk = h & 3;
        for (int t = 0; t < 2; ++t) {              // one 16-token tile at a time (register pressure)
            const bool krow = (kmask[t] >> tk) & 1u;
            const bf16_t *ksrc = kc + kblk[t] * kBlockElems + tk * 32 + 8 * g;
            const bf16_t *vblk = vc + kblk[t] * kBlockElems;
            f32x4 sc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < 8; ++s) {
                const bf16x8 kf = krow ? *reinterpret_cast<const bf16x8 *>(ksrc + s * 128) : bf16x8{};
                // dims d0 .. d0+7 of token tk: 64 B = 8 dims x 4 tokens, [dim][token]
                const bf16_t *vsrc = vblk + (32 * s + 8 * g) * kBlock;
                uint32_t wv[4];
                for (int m = 0; m < 4; ++m) {
                    const u32x4 w = *reinterpret_cast<const u32x4 *>(vsrc + 8 * m);
                    const int sh = 16 * (tk & 1);
                    const uint32_t lo = (w[tk >> 1] >> sh) & 0xFFFFu;
                    const uint32_t hi = (w[2 + (tk >> 1)] >> sh) & 0xFFFFu;
                    wv[m] = krow ? (lo | (hi << 16)) : 0u;
                }
                const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{wv[0], wv[1], wv[2], wv[3]});
                *reinterpret_cast<bf16x8 *>(&kt[16 * t + h][32 * s + 8 * g]) = kf;
                // S^T, dP^T: lane holds tokens 0..3 of entry lb + 4t + g (chunk tokens 16t + 4g + j) for head h
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], sc, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, dof[s], dp, 0, 0, 0);
            }
            for (int j = 0; j < 4; ++j) {
                const bool valid = ((omask[t] >> j) & 1u) && h < kGroup;
                const float pj = valid ? exp2f(sc[j] * c2 - lse2) : 0.f;
                const float ds = valid ? pj * (dp[j] - Dh) : 0.f;
                const int tok = 16 * t + 4 * g + j;
                pT[tok][h] = f32_to_bf16(pj);
                sT[tok][h] = f32_to_bf16(ds);
                sH[h][tok] = f32_to_bf16(ds);
            }
        }
        __syncthreads();
        // dV += P^T dO and dK~ += sigma dS^T Q~: 16x16x16 tiles, rows = chunk tokens, cols = dims
        for (int t = 0; t < 2; ++t) {
            const bf16x4 pa = *reinterpret_cast<const bf16x4 *>(&pT[16 * t + h][4 * g]);
            const bf16x4 sa = *reinterpret_cast<const bf16x4 *>(&sT[16 * t + h][4 * g]);
            const bool ev = omask[t] != 0u;
            const int64_t tok0 = kBlock * oblk[t];
            for (int n = 0; n < 16; ++n) {
                const bf16x4 ob = *reinterpret_cast<const bf16x4 *>(&oT[16 * n + h][4 * g]);
                const bf16x4 qb = *reinterpret_cast<const bf16x4 *>(&qT[16 * n + h][4 * g]);
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const f32x4 av = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, ob, zero, 0, 0, 0);
                const f32x4 ak = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(sa, qb, zero, 0, 0, 0);
                if (!ev) continue;
                for (int j = 0; j < 4; ++j) {
                    if (!((omask[t] >> j) & 1u)) continue;
                    const int64_t idx = ((b * L + tok0 + j) * kKVHeads + grp) * kHeadDim + 16 * n + h;
                    atomicAdd(dv + idx, av[j]);
                    atomicAdd(dk + idx, sigma * ak[j]);
                }
            }
        }
        // dQ~ += dS K~: 16x16x32 tiles, rows = heads, cols = dims, k = the chunk's 32 tokens
        const bf16x8 sa8 = *reinterpret_cast<const bf16x8 *>(&sH[h][8 * g]);
        for (int n = 0; n < 16; ++n) {
            uint32_t kw[4];
            for (int m = 0; m < 4; ++m)
                kw[m] = static_cast<uint32_t>(kt[8 * g + 2 * m][16 * n + h]) |
                        (static_cast<uint32_t>(kt[8 * g + 2 * m + 1][16 * n + h]) << 16);
            dqa[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sa8, __builtin_bit_cast(bf16x8, u32x4{kw[0], kw[1], kw[2], kw[3]}),
                                                             dqa[n], 0, 0, 0);
        }
        __syncthreads();
    }
    // dq = sigma R(p)^T dQ~: lane holds dims 16n + h of heads 4g + j; the rotary
    // partner of dim d < 32 (tile n < 2) is dim d + 32 (tile n + 2), same lane
    const float *cs = tab.cos + pos * kPairs;
    const float *sn = tab.sin + pos * kPairs;
    for (int n = 0; n < 2; ++n) {
        const int d = 16 * n + h;
        for (int j = 0; j < 4; ++j) {
            const float a = dqa[n][j], bb = dqa[n + 2][j];
            dqa[n][j] = a * cs[d] + bb * sn[d];
            dqa[n + 2][j] = bb * cs[d] - a * sn[d];
        }
    }
    for (int j = 0; j < 4; ++j) {
        const int head = 4 * g + j;
        if (head >= kGroup) continue;
        float *dst = dq + (row * kQHeads + grp * kGroup + head) * kHeadDim;
        for (int n = 0; n < 16; ++n) dst[16 * n + h] = sigma * dqa[n][j];
    }
}

// dk[b][t][g] = R(t)^T dK~[b][t][g] in place (dims 0..63), one thread per
// (token, group, rotary pair).
__global__ __launch_bounds__(256) void dk_unrotate_kernel(Tables tab, int32_t B, int64_t L, float *__restrict__ dk)
{
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (gid >= static_cast<int64_t>(B) * L * kKVHeads * kPairs) return;
    const int d = static_cast<int>(gid % kPairs);
    const int64_t rg = gid / kPairs;                   // (b, t, g)
    const int64_t t = (rg / kKVHeads) % L;
    float *x = dk + rg * kHeadDim;
    const float c = tab.cos[t * kPairs + d], s = tab.sin[t * kPairs + d];
    const float a = x[d], bb = x[d + kPairs];
    x[d] = a * c + bb * s;
    x[d + kPairs] = bb * c - a * s;
}

// Rows per launch of the indexer-loss forward walk (each query walks its
// blocks in ascending order; short launches keep the work-groups of a launch
// in step, as in the prefill walk).
constexpr int64_t kTrainLaunchRows = 4096;

hipError_t launch_attend_backward(const Tables &tab, hipStream_t st, int32_t B, int64_t L, int64_t nblk_cap, int budget,
                                  float sigma, const bf16_t *q, const bf16_t *k_cache, const bf16_t *v_cache,
                                  const int32_t *block_idx, const bf16_t *out, const bf16_t *dout, const float *stats,
                                  float *dq, float *dk, float *dv)
{
    if (L <= 0) return hipSuccess;
    // One launch: bound by its fp32 atomics, this walk measured 2% slower in
    // short launches.
    hipLaunchKernelGGL(attend_backward_kernel, dim3(static_cast<unsigned>(L), kKVHeads, static_cast<unsigned>(B)),
                       dim3(64), 0, st, tab, L, int64_t(0), nblk_cap, budget, sigma * kLog2e, sigma, q, k_cache, v_cache,
                       block_idx, out, dout, stats, dq, dk, dv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = static_cast<int64_t>(B) * L * kKVHeads * kPairs;
    hipLaunchKernelGGL(dk_unrotate_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, st, tab, B, L,
                       dk);
    return hipGetLastError();
}

hipError_t launch_train_kl(const Tables &tab, hipStream_t st, bool backward, int32_t B, int64_t L, int64_t nblk_cap,
                           int budget, float sigma, const bf16_t *q, const bf16_t *k_cache, const bf16_t *kbar,
                           const bf16_t *qrot, const int32_t *block_idx, float *stats, float *kl, const float *dkl,
                           float *dq_idx, float *dkbar)
{
    // The loss forward in short launches; its backward (bound by the pooled-key
    // gradient's atomics) in one, which measured 2% faster.
    const int64_t step = backward ? L : kTrainLaunchRows;
    for (int64_t r = 0; r < L; r += step) {
        const int64_t n = (r + step < L) ? step : L - r;
        dim3 grid(static_cast<unsigned>(n), static_cast<unsigned>(B));
        if (backward)
            hipLaunchKernelGGL(train_kl_kernel<true>, grid, dim3(128), 0, st, tab, L, r, nblk_cap, budget,
                               sigma * kLog2e, q, k_cache, kbar, qrot, block_idx, stats, kl, dkl, dq_idx, dkbar);
        else
            hipLaunchKernelGGL(train_kl_kernel<false>, grid, dim3(128), 0, st, tab, L, r, nblk_cap, budget,
                               sigma * kLog2e, q, k_cache, kbar, qrot, block_idx, stats, kl, dkl, dq_idx, dkbar);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
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
