// Device helpers shared by the sparse-attention kernels (inference and
// training): the query fragments of one (query, KV group) rotated on load, and
// the walk over a query's token list (selected blocks, then tail blocks).
#pragma once

#include "qsa_common.h"

namespace qsa {

constexpr int kChunkBlocks = 8;                  // 32 tokens per step
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Per-query training statistics (floats): the 24 heads' log-sum-exp of their
// scaled logits, then ln of the teacher's block-weight sum, then the
// log-sum-exp of the student's scores; the rest is zero.
constexpr int kTrainStats = 32;

// Q~^T fragments of one (query, KV group): lane (h = l%16, g = l/16) holds, for
// k-step s, dims 32s + 8g .. +7 of head 12*grp + h, rotated at `pos` (heads
// 12..15 of the 16-wide tile are zero).
__device__ __forceinline__ void load_q_frags(const bf16_t *qrow /*[24][256] of this token*/, int grp, int64_t pos,
                                             const Tables &tab, bf16x8 (&qf)[8])
{
    const int lane = threadIdx.x & 63;
    const int h = lane & 15, g = lane >> 4;
    if (h >= kGroup) {
        for (int s = 0; s < 8; ++s) qf[s] = bf16x8{};
        return;
    }
    const bf16_t *src = qrow + (grp * kGroup + h) * kHeadDim + 8 * g;
    u32x4 x[8];
    for (int s = 0; s < 8; ++s) x[s] = *reinterpret_cast<const u32x4 *>(src + 32 * s);
    // rotary pairs (j, j + 32), j = 8g + e: k-step 0 holds x_j, k-step 1 holds x_{j+32}
    const float *cs = tab.cos + pos * kPairs + 8 * g;
    const float *sn = tab.sin + pos * kPairs + 8 * g;
    uint32_t w0[4], w1[4];
    for (int i = 0; i < 4; ++i) {
        float r0[2], r1[2];
        for (int e = 0; e < 2; ++e) {
            float a = __uint_as_float(e ? (x[0][i] & 0xFFFF0000u) : (x[0][i] << 16));
            float b = __uint_as_float(e ? (x[1][i] & 0xFFFF0000u) : (x[1][i] << 16));
            rotate_pair(a, b, cs[2 * i + e], sn[2 * i + e]);
            r0[e] = a;
            r1[e] = b;
        }
        w0[i] = pack_bf16x2(r0[0], r0[1]);
        w1[i] = pack_bf16x2(r1[0], r1[1]);
    }
    x[0] = u32x4{w0[0], w0[1], w0[2], w0[3]};
    x[1] = u32x4{w1[0], w1[1], w1[2], w1[3]};
    for (int s = 0; s < 8; ++s) qf[s] = __builtin_bit_cast(bf16x8, x[s]);
}

// Block id and valid-token mask (bit t = token t valid) of list entry li.
// The list is the n_sel selected blocks (only ids in [0, o0) count), then the
// tail blocks o0 .. o, whole except the query's own block o, whose tokens run
// to own_last.  A selection made at the query itself has o0 = o (the tail is
// the own block alone); one reused from an earlier position has o0 = its own
// block there.
// Entry li of the list from its (already loaded) selection value id, branch-free.
__device__ __forceinline__ void entry_from_id(int64_t id, int n_sel, int64_t o0, int64_t o, int li, int own_last,
                                              int64_t &blk, uint32_t &tmask)
{
    const bool in_sel = li < n_sel;
    const int64_t tb = o0 + (li - n_sel);
    const bool in_tail = !in_sel && tb <= o;
    const bool ok = in_sel && id >= 0 && id < o0;
    const uint32_t tail_mask = (tb == o) ? (1u << (own_last + 1)) - 1u : 0xFu;
    blk = ok ? id : (in_tail ? tb : 0);
    tmask = ok ? 0xFu : (in_tail ? tail_mask : 0u);
}

// The selection value entry li reads (clamped into the list; ignored past it).
// sel holds the entries from sel_off on (sel_off <= li for every li read).
__device__ __forceinline__ int32_t entry_id(const int32_t *sel, int n_sel, int li, int sel_off) {
    return sel[(li < n_sel ? li : sel_off) - sel_off];
}

template <bool kBranchFree = false>
__device__ __forceinline__ void list_entry(const int32_t *sel, int sel_off, int n_sel, int64_t o0, int64_t o, int li,
                                           int own_last, int64_t &blk, uint32_t &tmask)
{
    if constexpr (kBranchFree) {
        // The list read unconditionally (index clamped into the list), no
        // branches: a chunk's entries are loaded together instead of one wait
        // each.  The prefill walk gains about 1%; the decode split kernel
        // measured slower with it.
        entry_from_id(entry_id(sel, n_sel, li, sel_off), n_sel, o0, o, li, own_last, blk, tmask);
    } else if (li < n_sel) {
        const int64_t id = sel[li - sel_off];
        const bool ok = id >= 0 && id < o0;
        blk = ok ? id : 0;
        tmask = ok ? 0xFu : 0u;
    } else if (li - n_sel <= o - o0) {
        blk = o0 + (li - n_sel);
        tmask = (blk == o) ? (1u << (own_last + 1)) - 1u : 0xFu;
    } else {
        blk = 0;
        tmask = 0u;
    }
}

// Chunks of a token list of n_sel selected blocks and tail blocks o0 .. o.
__device__ __forceinline__ int list_chunks(int n_sel, int64_t o0, int64_t o) {
    return static_cast<int>((n_sel + (o - o0) + 1 + kChunkBlocks - 1) / kChunkBlocks);
}

}  // namespace qsa
