// Sparse core attention over the selected micro-blocks (PyTorchKR post
// "Qwen3.8-Flash-Next, 1/9의 학습 비용으로 …", section "QSA: 인덱서 자체의 비용을
// 줄이는 희소 어텐션": GQA over the top blocks; the tail tokens of the last
// incomplete block are always included; spec table: 24 query heads, 2 KV
// heads, head dim 256, RoPE on 64 dims).
//
// A wave walks (query, KV head) pairs -- two in turn in the prefill kernel, one
// in the training and decode kernels: the 12 query heads of the group share
// every gathered K~/V micro-block.  The token list of query p is the
// selected blocks (ascending) followed by its own block 4*floor(p/4) .. p; it is
// walked in chunks of 8 blocks (32 tokens).
//
// Matrix-core layout (v_mfma_f32_16x16x32_bf16, 16x16 output, lane l holds
// column l%16 and rows 4*(l/16) .. +3):
//   S^T  = K~ . Q~^T   A = 16 tokens x 32 dims of K~ (straight 16-byte loads
//                      from the blocked cache), B = Q~^T (head l%16), so each
//                      lane ends with 4 tokens of one head;
//   O^T += V^T . P^T   B = P^T comes straight from the S^T registers (the
//                      contraction index is permuted to match), A = V^T from
//                      the blocked V cache ([dim][4 tokens] per block, 8-byte
//                      loads), and every O^T accumulator of a lane belongs to
//                      the same head as its softmax state -- no shuffles.
// Softmax is online in fp32 (base-2 exponentials, max over the 4 lane groups
// by two xor-shuffles); P is rounded to bf16 for the PV product.
#include "qsa_common.h"
#include "attend_parts.h"

namespace qsa {

struct RowState {
    float m;        // running max of the raw logits of head l%16 (same in the 4 lane groups)
    float l;        // this lane's partial softmax denominator
    f32x4 o[16];    // O^T: dims 16n + 4*(l/16) + j of head l%16
};

// Walk chunks [c_lo, c_hi) of one (query, group) token list; sel holds the
// selection from entry sel_off on.
template <bool kBranchFree>
__device__ __forceinline__ void attend_chunks(const bf16x8 (&qf)[8], const bf16_t *__restrict__ kc,
                                              const bf16_t *__restrict__ vc, const int32_t *__restrict__ sel,
                                              int sel_off, int n_sel, int64_t o0, int64_t o, int own_last, int c_lo,
                                              int c_hi, float c2, RowState &st)
{
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;           // K-load token row / V-load dim
    const int g = lane >> 4;
    for (int c = c_lo; c < c_hi; ++c) {
        const int lb = kChunkBlocks * c;
        // ---- gather K~ (A operand of S^T): tile t, token row r -> list entry lb + 4t + r/4
        int64_t kblk[2];
        uint32_t kmask[2];
        for (int t = 0; t < 2; ++t) list_entry<kBranchFree>(sel, sel_off, n_sel, o0, o, lb + 4 * t + (r >> 2), own_last, kblk[t], kmask[t]);
        bf16x8 kf[2][8];
        for (int t = 0; t < 2; ++t) {
            const bf16_t *src = kc + kblk[t] * kBlockElems + (r & 3) * 32 + 8 * g;
            for (int s = 0; s < 8; ++s) kf[t][s] = *reinterpret_cast<const bf16x8 *>(src + s * 128);
        }
        // ---- gather V (A operand of O^T): list entries lb + g and lb + 4 + g, dim 16n + r
        int64_t vblk[2];
        uint32_t vmask[2];
        for (int t = 0; t < 2; ++t) list_entry<kBranchFree>(sel, sel_off, n_sel, o0, o, lb + 4 * t + g, own_last, vblk[t], vmask[t]);
        u32x2 vraw[16][2];
        for (int t = 0; t < 2; ++t) {
            const bf16_t *src = vc + vblk[t] * kBlockElems + r * kBlock;
            for (int n = 0; n < 16; ++n) vraw[n][t] = *reinterpret_cast<const u32x2 *>(src + 16 * n * kBlock);
        }
        // ---- S^T = K~ . Q~^T
        f32x4 sc[2];
        for (int t = 0; t < 2; ++t) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t][s], qf[s], acc, 0, 0, 0);
            sc[t] = acc;
        }
        // lane holds tokens j = 0..3 of list entry lb + 4t + g for head r
        float cmax = -INFINITY;
        for (int t = 0; t < 2; ++t) {
            for (int j = 0; j < 4; ++j) {
                if (!((vmask[t] >> j) & 1u)) sc[t][j] = -INFINITY;
                cmax = fmaxf(cmax, sc[t][j]);
            }
        }
        cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
        const float m_new = fmaxf(st.m, cmax);
        // While every token so far was masked m_new is -inf; 0 then serves as
        // the reference so that alpha and p come out 0 instead of NaN.
        const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f((st.m - m_ref) * c2);
        st.m = m_new;
        uint32_t pw[4];
        float psum = 0.f;
        for (int t = 0; t < 2; ++t) {
            float p[4];
            for (int j = 0; j < 4; ++j) {
                p[j] = exp2f((sc[t][j] - m_ref) * c2);
            }
            pw[2 * t] = pack_bf16x2(p[0], p[1]);
            pw[2 * t + 1] = pack_bf16x2(p[2], p[3]);
            for (int j = 0; j < 4; ++j) psum += bf16_to_f32(f32_to_bf16(p[j]));
        }
        st.l = st.l * alpha + psum;
        const bf16x8 pf = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
        // ---- O^T += V^T . P^T  (zero the V of masked tokens: their cache slots may hold anything)
        for (int n = 0; n < 16; ++n) {
            u32x2 lo = vraw[n][0], hi = vraw[n][1];
            const uint32_t m0 = vmask[0], m1 = vmask[1];
            lo[0] &= ((m0 & 1u) ? 0xFFFFu : 0u) | ((m0 & 2u) ? 0xFFFF0000u : 0u);
            lo[1] &= ((m0 & 4u) ? 0xFFFFu : 0u) | ((m0 & 8u) ? 0xFFFF0000u : 0u);
            hi[0] &= ((m1 & 1u) ? 0xFFFFu : 0u) | ((m1 & 2u) ? 0xFFFF0000u : 0u);
            hi[1] &= ((m1 & 4u) ? 0xFFFFu : 0u) | ((m1 & 8u) ? 0xFFFF0000u : 0u);
            const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
            f32x4 acc = st.o[n];
            for (int j = 0; j < 4; ++j) acc[j] *= alpha;
            st.o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc, 0, 0, 0);
        }
    }
}

__device__ __forceinline__ void init_state(RowState &st) {
    st.m = -INFINITY;
    st.l = 0.f;
    for (int n = 0; n < 16; ++n) st.o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Prefill work-group order: all queries of KV group 0, then all of group 1;
// wave w of work-group x takes rows 2s and 2s+1, s = 4x' + w.  The work-groups
// resident at any time then gather from one group's cache (half of the K~/V
// bytes), so more of the blocks they ask for are still in the L2: fewer bytes
// cross to HBM.
__device__ __forceinline__ void prefill_pair_slot(int64_t L, int wave, int64_t &i0, int &grp)
{
    const int64_t nt = (L + 7) / 8;
    const int64_t x = blockIdx.x;
    grp = x >= nt ? 1 : 0;
    i0 = ((x - grp * nt) * 4 + wave) * 2;
}

// Normalise a finished walk and store the 12 heads of (row, group).
__device__ __forceinline__ void store_row(const RowState &st, bf16_t *__restrict__ out_row /*[24][256]*/, int grp)
{
    const int lane = threadIdx.x & 63;
    float lt = st.l + __shfl_xor(st.l, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = 1.0f / lt;
    const int h = lane & 15, g = lane >> 4;
    if (h < kGroup) {
        bf16_t *dst = out_row + (grp * kGroup + h) * kHeadDim + 4 * g;
        for (int n = 0; n < 16; ++n) {
            u32x2 w = u32x2{pack_bf16x2(st.o[n][0] * inv, st.o[n][1] * inv),
                            pack_bf16x2(st.o[n][2] * inv, st.o[n][3] * inv)};
            *reinterpret_cast<u32x2 *>(dst + 16 * n) = w;
        }
    }
}

// Prefill: 4 waves per work-group, each walking the token lists of two
// neighbouring queries of one KV group, one chunk of each in turn, each into
// its own softmax state (a query's chunks in ascending order, as a walk of
// its own would take them, so the output does not depend on the pairing).
// Two walks per wave put twice as many walks in progress on a CU for the same
// bytes in flight, each advancing at half the pace.
__global__ __launch_bounds__(256) void attend_prefill_kernel(
    Tables tab, int64_t L, int64_t row0, int64_t ld, int64_t q_offset, int64_t nblk_cap, int budget, float c2,
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k_cache, const bf16_t *__restrict__ v_cache,
    const int32_t *__restrict__ block_idx, bf16_t *__restrict__ out)
{
    const int wave = threadIdx.x >> 6;
    const int64_t b = blockIdx.y;
    int64_t il;
    int grp;
    prefill_pair_slot(L, wave, il, grp);
    if (il >= L) return;
    const bool two = il + 1 < L;          // a ragged launch may end on a lone row
    const int64_t i0 = row0 + il, i1 = two ? i0 + 1 : i0;
    const int64_t pos0 = q_offset + i0, pos1 = q_offset + i1;
    const int64_t o0 = pos0 / kBlock, o1 = pos1 / kBlock;
    const int own0 = static_cast<int>(pos0 - o0 * kBlock), own1 = static_cast<int>(pos1 - o1 * kBlock);
    const int nsel0 = static_cast<int>(o0 < budget ? o0 : budget), nsel1 = static_cast<int>(o1 < budget ? o1 : budget);
    const int nch0 = list_chunks(nsel0, o0, o0), nch1 = two ? list_chunks(nsel1, o1, o1) : 0;

    bf16x8 qf0[8], qf1[8];
    load_q_frags(q + (b * ld + i0) * kQHeads * kHeadDim, grp, pos0, tab, qf0);
    load_q_frags(q + (b * ld + i1) * kQHeads * kHeadDim, grp, pos1, tab, qf1);
    const bf16_t *kc = k_cache + kcache_block_base(b, grp, 0, nblk_cap);
    const bf16_t *vc = v_cache + kcache_block_base(b, grp, 0, nblk_cap);
    const int32_t *sel0 = block_idx + (b * ld + i0) * budget;
    const int32_t *sel1 = block_idx + (b * ld + i1) * budget;

    RowState st0, st1;
    init_state(st0);
    init_state(st1);
    const int nmax = nch0 > nch1 ? nch0 : nch1;
    for (int c = 0; c < nmax; ++c) {
        // the two chunks are not interleaved by the scheduler: one chunk's
        // gathers and logits at a time fit the register file with both states
        if (c < nch0) attend_chunks<true>(qf0, kc, vc, sel0, 0, nsel0, o0, o0, own0, c, c + 1, c2, st0);
        __builtin_amdgcn_sched_barrier(0);
        if (c < nch1) attend_chunks<true>(qf1, kc, vc, sel1, 0, nsel1, o1, o1, own1, c, c + 1, c2, st1);
        __builtin_amdgcn_sched_barrier(0);
    }
    store_row(st0, out + (b * ld + i0) * kQHeads * kHeadDim, grp);
    if (two) store_row(st1, out + (b * ld + i1) * kQHeads * kHeadDim, grp);
}

// Prefill attention of the training forward: the walk of attend_prefill_kernel
// (q_offset 0) over rows row0 .. row0+n-1 of L, and each head's natural-log
// log-sum-exp of its scaled logits over T(p), sigma*m + ln(l), stored at
// stats[row*32 + head] for the teacher of the indexer loss.  The walk is
// written out again rather than shared through an inlined function: the
// prefill kernel built from a shared function scheduled differently and
// measured 1% slower (85.4-85.5 against 84.45-84.5 ms at 262,144 tokens).
__device__ __forceinline__ void store_row_stats(const RowState &st, bf16_t *__restrict__ out_row /*[24][256]*/,
                                                int grp, float c2, float *__restrict__ stats_row /*[32]*/)
{
    const int lane = threadIdx.x & 63;
    float lt = st.l + __shfl_xor(st.l, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = 1.0f / lt;
    const int h = lane & 15, g = lane >> 4;
    if (h < kGroup) {
        bf16_t *dst = out_row + (grp * kGroup + h) * kHeadDim + 4 * g;
        for (int n = 0; n < 16; ++n) {
            u32x2 w = u32x2{pack_bf16x2(st.o[n][0] * inv, st.o[n][1] * inv),
                            pack_bf16x2(st.o[n][2] * inv, st.o[n][3] * inv)};
            *reinterpret_cast<u32x2 *>(dst + 16 * n) = w;
        }
        if (g == 0) stats_row[grp * kGroup + h] = (st.m * c2 + log2f(lt)) * kLn2;
    }
}

__global__ __launch_bounds__(256) void attend_stats_kernel(
    Tables tab, int64_t L, int64_t n, int64_t row0, int64_t nblk_cap, int budget, float c2,
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k_cache, const bf16_t *__restrict__ v_cache,
    const int32_t *__restrict__ block_idx, bf16_t *__restrict__ out, float *__restrict__ stats)
{
    const int wave = threadIdx.x >> 6;
    const int64_t b = blockIdx.y;
    int64_t il;
    int grp;
    prefill_pair_slot(n, wave, il, grp);
    if (il >= n) return;
    const bool two = il + 1 < n;
    const int64_t i0 = row0 + il, i1 = two ? i0 + 1 : i0;     // rows of L; positions = rows
    const int64_t o0 = i0 / kBlock, o1 = i1 / kBlock;
    const int own0 = static_cast<int>(i0 - o0 * kBlock), own1 = static_cast<int>(i1 - o1 * kBlock);
    const int nsel0 = static_cast<int>(o0 < budget ? o0 : budget), nsel1 = static_cast<int>(o1 < budget ? o1 : budget);
    const int nch0 = list_chunks(nsel0, o0, o0), nch1 = two ? list_chunks(nsel1, o1, o1) : 0;

    bf16x8 qf0[8], qf1[8];
    load_q_frags(q + (b * L + i0) * kQHeads * kHeadDim, grp, i0, tab, qf0);
    load_q_frags(q + (b * L + i1) * kQHeads * kHeadDim, grp, i1, tab, qf1);
    const bf16_t *kc = k_cache + kcache_block_base(b, grp, 0, nblk_cap);
    const bf16_t *vc = v_cache + kcache_block_base(b, grp, 0, nblk_cap);
    const int32_t *sel0 = block_idx + (b * L + i0) * budget;
    const int32_t *sel1 = block_idx + (b * L + i1) * budget;

    RowState st0, st1;
    init_state(st0);
    init_state(st1);
    const int nmax = nch0 > nch1 ? nch0 : nch1;
    for (int c = 0; c < nmax; ++c) {
        if (c < nch0) attend_chunks<true>(qf0, kc, vc, sel0, 0, nsel0, o0, o0, own0, c, c + 1, c2, st0);
        __builtin_amdgcn_sched_barrier(0);
        if (c < nch1) attend_chunks<true>(qf1, kc, vc, sel1, 0, nsel1, o1, o1, own1, c, c + 1, c2, st1);
        __builtin_amdgcn_sched_barrier(0);
    }
    store_row_stats(st0, out + (b * L + i0) * kQHeads * kHeadDim, grp, c2, stats + (b * L + i0) * kTrainStats);
    if (two) store_row_stats(st1, out + (b * L + i1) * kQHeads * kHeadDim, grp, c2, stats + (b * L + i1) * kTrainStats);
}

// The decode walk: the arithmetic of attend_chunks with the gathers of the
// next chunk issued while the current one computes -- its K~ once the current
// logits are formed, its V after the current PV product -- so that a wave
// keeps a chunk's worth of loads in flight through its walk with no more
// registers than one chunk needs.  The gathers are non-temporal loads: a
// decode step reads each selected block once per (sequence, KV group).  (The
// prefill walk keeps plain loads: there the walks that run together reuse each
// other's blocks through the L2.)
__device__ __forceinline__ void fetch_chunk_k(const bf16_t *__restrict__ kc, const int32_t *__restrict__ sel,
                                              int sel_off, int n_sel, int64_t o0, int64_t o, int own_last, int c,
                                              bf16x8 (&kf)[2][8])
{
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int lb = kChunkBlocks * c;
    for (int t = 0; t < 2; ++t) {
        int64_t blk;
        uint32_t m;
        list_entry<false>(sel, sel_off, n_sel, o0, o, lb + 4 * t + (r >> 2), own_last, blk, m);
        const bf16_t *src = kc + blk * kBlockElems + (r & 3) * 32 + 8 * g;
        for (int s = 0; s < 8; ++s)
            kf[t][s] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(src + s * 128));
    }
}

__device__ __forceinline__ void fetch_chunk_v(const bf16_t *__restrict__ vc, const int32_t *__restrict__ sel,
                                              int sel_off, int n_sel, int64_t o0, int64_t o, int own_last, int c,
                                              u32x2 (&vraw)[16][2], uint32_t (&vmask)[2])
{
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int lb = kChunkBlocks * c;
    for (int t = 0; t < 2; ++t) {
        int64_t blk;
        list_entry<false>(sel, sel_off, n_sel, o0, o, lb + 4 * t + g, own_last, blk, vmask[t]);
        const bf16_t *src = vc + blk * kBlockElems + r * kBlock;
        for (int n = 0; n < 16; ++n)
            vraw[n][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(src + 16 * n * kBlock));
    }
}

// One chunk of the decode walk; with kNext the next chunk's K~ is fetched
// after the logits and its V after the PV product.  The last chunk of a walk
// is a separate instance without fetches, so that every instance is straight
// code and the wait before a product counts only the loads it needs.
template <bool kNext>
__device__ __forceinline__ void decode_chunk(const bf16x8 (&qf)[8], const bf16_t *__restrict__ kc,
                                             const bf16_t *__restrict__ vc, const int32_t *__restrict__ sel,
                                             int sel_off, int n_sel, int64_t o0, int64_t o, int own_last, int c,
                                             float c2, bf16x8 (&kf)[2][8], u32x2 (&vraw)[16][2],
                                             uint32_t (&vmask)[2], RowState &st)
{
    // ---- S^T = K~ . Q~^T, then the next chunk's K~ into the freed registers
    f32x4 sc[2];
    for (int t = 0; t < 2; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t][s], qf[s], acc, 0, 0, 0);
        sc[t] = acc;
    }
    if constexpr (kNext) fetch_chunk_k(kc, sel, sel_off, n_sel, o0, o, own_last, c + 1, kf);
    // lane holds tokens j = 0..3 of list entry 8c + 4t + g for head l%16
    float cmax = -INFINITY;
    for (int t = 0; t < 2; ++t) {
        for (int j = 0; j < 4; ++j) {
            if (!((vmask[t] >> j) & 1u)) sc[t][j] = -INFINITY;
            cmax = fmaxf(cmax, sc[t][j]);
        }
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(st.m, cmax);
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;     // as in attend_chunks
    const float alpha = exp2f((st.m - m_ref) * c2);
    st.m = m_new;
    uint32_t pw[4];
    float psum = 0.f;
    for (int t = 0; t < 2; ++t) {
        float p[4];
        for (int j = 0; j < 4; ++j) p[j] = exp2f((sc[t][j] - m_ref) * c2);
        pw[2 * t] = pack_bf16x2(p[0], p[1]);
        pw[2 * t + 1] = pack_bf16x2(p[2], p[3]);
        for (int j = 0; j < 4; ++j) psum += bf16_to_f32(f32_to_bf16(p[j]));
    }
    st.l = st.l * alpha + psum;
    const bf16x8 pf = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
    // ---- O^T += V^T . P^T (masked tokens' V zeroed), then the next chunk's V
    for (int n = 0; n < 16; ++n) {
        u32x2 lo = vraw[n][0], hi = vraw[n][1];
        const uint32_t m0 = vmask[0], m1 = vmask[1];
        lo[0] &= ((m0 & 1u) ? 0xFFFFu : 0u) | ((m0 & 2u) ? 0xFFFF0000u : 0u);
        lo[1] &= ((m0 & 4u) ? 0xFFFFu : 0u) | ((m0 & 8u) ? 0xFFFF0000u : 0u);
        hi[0] &= ((m1 & 1u) ? 0xFFFFu : 0u) | ((m1 & 2u) ? 0xFFFF0000u : 0u);
        hi[1] &= ((m1 & 4u) ? 0xFFFFu : 0u) | ((m1 & 8u) ? 0xFFFF0000u : 0u);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        f32x4 acc = st.o[n];
        for (int j = 0; j < 4; ++j) acc[j] *= alpha;
        st.o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc, 0, 0, 0);
    }
    if constexpr (kNext) fetch_chunk_v(vc, sel, sel_off, n_sel, o0, o, own_last, c + 1, vraw, vmask);
}

__device__ __forceinline__ void decode_walk(const bf16x8 (&qf)[8], const bf16_t *__restrict__ kc,
                                            const bf16_t *__restrict__ vc, const int32_t *__restrict__ sel,
                                            int sel_off, int n_sel, int64_t o0, int64_t o, int own_last, int c_lo,
                                            int c_hi, float c2, RowState &st)
{
    if (c_lo >= c_hi) return;
    bf16x8 kf[2][8];
    u32x2 vraw[16][2];
    uint32_t vmask[2];
    fetch_chunk_k(kc, sel, sel_off, n_sel, o0, o, own_last, c_lo, kf);
    fetch_chunk_v(vc, sel, sel_off, n_sel, o0, o, own_last, c_lo, vraw, vmask);
    int c = c_lo;
    for (; c + 1 < c_hi; ++c)
        decode_chunk<true>(qf, kc, vc, sel, sel_off, n_sel, o0, o, own_last, c, c2, kf, vraw, vmask, st);
    decode_chunk<false>(qf, kc, vc, sel, sel_off, n_sel, o0, o, own_last, c, c2, kf, vraw, vmask, st);
}

// Decode, split over the token list: one wave per (split, group, sequence)
// writes its unnormalised partial (m, l, O) for the 12 heads.  With sel_pos
// (a reused selection) the list is block_idx as selected at position
// p0 = sel_pos[b] (clamped to [0, p]) followed by every block from p0's own
// block up to the query's.
__global__ __launch_bounds__(64) void attend_decode_split_kernel(
    Tables tab, const int32_t *__restrict__ cache_len, const int32_t *__restrict__ sel_pos, int64_t ctx_bound,
    int64_t nblk_cap, int budget, int nsplit, float c2,
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k_cache, const bf16_t *__restrict__ v_cache,
    const int32_t *__restrict__ block_idx, float *__restrict__ part_o, float *__restrict__ part_ml)
{
    const int lane = threadIdx.x & 63;
    const int split = blockIdx.x;
    const int grp = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int64_t pos = decode_pos(cache_len, b, ctx_bound);
    const int64_t o = pos / kBlock;
    const int own_last = static_cast<int>(pos - o * kBlock);
    const int64_t o0 = sel_pos ? decode_pos(sel_pos, b, pos) / kBlock : o;
    const int n_sel = static_cast<int>(o0 < budget ? o0 : budget);
    const int nchunks = list_chunks(n_sel, o0, o);
    const int per = (nchunks + nsplit - 1) / nsplit;
    const int c_lo = split * per;
    const int c_hi = (c_lo + per < nchunks) ? c_lo + per : nchunks;

    // The split's part of the selection, staged in LDS once: the walk then
    // reads its entries without a global round trip before each chunk's gathers.
    __shared__ int32_t lsel[kMaxBudget];
    const int e_lo = kChunkBlocks * c_lo;
    const int e_hi = (kChunkBlocks * c_hi < n_sel) ? kChunkBlocks * c_hi : n_sel;
    for (int e = e_lo + lane; e < e_hi; e += 64) lsel[e - e_lo] = block_idx[b * budget + e];
    __syncthreads();

    RowState st;
    init_state(st);
    if (c_lo < c_hi) {
        bf16x8 qf[8];
        load_q_frags(q + b * kQHeads * kHeadDim, grp, pos, tab, qf);
        const bf16_t *kc = k_cache + kcache_block_base(b, grp, 0, nblk_cap);
        const bf16_t *vc = v_cache + kcache_block_base(b, grp, 0, nblk_cap);
        decode_walk(qf, kc, vc, lsel, e_lo, n_sel, o0, o, own_last, c_lo, c_hi, c2, st);
    }
    float lt = st.l + __shfl_xor(st.l, 16);
    lt += __shfl_xor(lt, 32);
    const int h = lane & 15, g = lane >> 4;
    if (h < kGroup) {
        const int64_t slot = ((b * kKVHeads + grp) * nsplit + split) * kGroup + h;
        float *dst = part_o + slot * kHeadDim + 4 * g;
        for (int n = 0; n < 16; ++n) *reinterpret_cast<f32x4 *>(dst + 16 * n) = st.o[n];
        if (g == 0) {
            part_ml[slot * 2] = st.m;
            part_ml[slot * 2 + 1] = lt;
        }
    }
}

// Merge the splits of one (sequence, head): 256 threads = one per dim.
__global__ __launch_bounds__(256) void attend_decode_merge_kernel(int nsplit, float c2,
                                                                  const float *__restrict__ part_o,
                                                                  const float *__restrict__ part_ml,
                                                                  bf16_t *__restrict__ out)
{
    constexpr int kMaxSplits = 32;
    __shared__ float ws_w[kMaxSplits], ws_l[kMaxSplits];
    const int d = threadIdx.x;
    const int head = blockIdx.x;                    // 0..23
    const int64_t b = blockIdx.y;
    const int grp = head / kGroup, h = head % kGroup;
    const int64_t slot0 = ((b * kKVHeads + grp) * nsplit) * kGroup + h;
    // split weights 2^{(m_s - m) c2}, one lane per split (0 for an empty split)
    if (d < 64) {
        const bool on = d < nsplit;
        const float ms = on ? part_ml[(slot0 + d * kGroup) * 2] : -INFINITY;
        const float ls = on ? part_ml[(slot0 + d * kGroup) * 2 + 1] : 0.f;
        float m = ms;
        for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
        if (d < kMaxSplits) {
            ws_w[d] = (on && ms != -INFINITY) ? exp2f((ms - m) * c2) : 0.f;
            ws_l[d] = (on && ms != -INFINITY) ? ls : -1.f;       // -1 marks a skipped split
        }
    }
    __syncthreads();
    // sums in split order; the partial rows are loaded eight splits at a time
    float l = 0.f, acc = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += 8) {
        float po[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            po[i] = (s0 + i < nsplit) ? part_o[(slot0 + (s0 + i) * kGroup) * kHeadDim + d] : 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (s0 + i >= nsplit || ws_l[s0 + i] < 0.f) continue;
            const float w = ws_w[s0 + i];
            l += ws_l[s0 + i] * w;
            acc += po[i] * w;
        }
    }
    out[(b * kQHeads + head) * kHeadDim + d] = f32_to_bf16(acc / l);
}

// ---------------------------------------------------------------- launchers
// Rows per launch of the prefill walk.  Every query walks its blocks in
// ascending order; the work-groups of one launch start together and walk in
// step, so at any time they gather from the same part of the cache and share
// what the L2 holds.  Over a long launch the later work-groups start at
// scattered times and that sharing is lost: at 262,144 tokens one launch over
// all rows took 114 ms, launches of 32,768 / 8,192 / 4,096 / 2,048 rows 105 /
// 89 / 85 / 84 ms, with bitwise the same output (one query per wave).  The
// walk with two queries per wave, in launches of 2,048 rows (one
// resident set of work-groups per KV group): 84.3-84.4 ms at 262,144 tokens
// against 85.1-85.4 ms for one query per wave in 4,096-row launches, with
// bitwise the same output.
constexpr int64_t kAttendPairLaunchRows = 2048;

hipError_t launch_attend_prefill(const Tables &tab, hipStream_t st, int32_t B, int64_t L, int64_t row0, int64_t ld,
                                 int64_t q_offset, int64_t nblk_cap, int budget, float sigma, const bf16_t *q,
                                 const bf16_t *k_cache, const bf16_t *v_cache, const int32_t *block_idx, bf16_t *out)
{
    for (int64_t r = 0; r < L; r += kAttendPairLaunchRows) {
        const int64_t n = (r + kAttendPairLaunchRows < L) ? kAttendPairLaunchRows : L - r;
        dim3 grid(static_cast<unsigned>(2 * ((n + 7) / 8)), static_cast<unsigned>(B));
        hipLaunchKernelGGL(attend_prefill_kernel, grid, dim3(256), 0, st, tab, n, row0 + r, ld, q_offset,
                           nblk_cap, budget, sigma * kLog2e, q, k_cache, v_cache, block_idx, out);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_attend_stats(const Tables &tab, hipStream_t st, int32_t B, int64_t L, int64_t nblk_cap, int budget,
                               float sigma, const bf16_t *q, const bf16_t *k_cache, const bf16_t *v_cache,
                               const int32_t *block_idx, bf16_t *out, float *stats)
{
    for (int64_t r = 0; r < L; r += kAttendPairLaunchRows) {     // as launch_attend_prefill
        const int64_t n = (r + kAttendPairLaunchRows < L) ? kAttendPairLaunchRows : L - r;
        dim3 grid(static_cast<unsigned>(2 * ((n + 7) / 8)), static_cast<unsigned>(B));
        hipLaunchKernelGGL(attend_stats_kernel, grid, dim3(256), 0, st, tab, L, n, r, nblk_cap, budget,
                           sigma * kLog2e, q, k_cache, v_cache, block_idx, out, stats);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_attend_decode(const Tables &tab, hipStream_t st, int32_t B, const int32_t *cache_len,
                                const int32_t *sel_pos, int64_t ctx_bound, int64_t nblk_cap, int budget, int nsplit,
                                float sigma, const bf16_t *q, const bf16_t *k_cache, const bf16_t *v_cache,
                                const int32_t *block_idx,
                                float *part_o, float *part_ml, bf16_t *out)
{
    if (B <= 0) return hipSuccess;
    const float c2 = sigma * kLog2e;
    hipLaunchKernelGGL(attend_decode_split_kernel, dim3(nsplit, kKVHeads, B), dim3(64), 0, st, tab, cache_len,
                       sel_pos, ctx_bound, nblk_cap, budget, nsplit, c2, q, k_cache, v_cache, block_idx, part_o, part_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attend_decode_merge_kernel, dim3(kQHeads, B), dim3(256), 0, st, nsplit, c2, part_o, part_ml,
                       out);
    return hipGetLastError();
}

}  // namespace qsa
