// Dense causal GQA attention over the K~/V caches: the dense baseline of the
// pages' module speed-ups (PyTorchKR post "Qwen3.8-Flash-Next, 1/9의 학습 비용으로
// …", section "QSA: 인덱서 자체의 비용을 줄이는 희소 어텐션", kernel-latency figure:
// QSA's indexer + sparse core attention against a dense paged GQA kernel).
// Query p attends every token 0..p; head h reads KV head h / 12; the same
// rotation, scale and precision as the sparse kernel (bf16 operands, fp32
// logits and softmax, P rounded to bf16 for the PV product, bf16 output).
//
// Flash-style tiling for gfx950.  A work-group (4 waves) owns 16 consecutive
// queries of one KV group; wave w owns queries 4w .. 4w+3 and their 12 heads:
// 48 (query, head) columns = 3 column tiles of 16.  The keys are walked in
// chunks of 32 (8 micro-blocks): the chunk's K~ and V are copied once into
// LDS -- already permuted into MFMA operand order, so every operand read is
// one conflict-free 16-byte LDS load per lane -- and shared by the 4 waves, so
// each gathered byte feeds 16 queries x 12 heads.  The next chunk is loaded
// into registers while the current one is computed (double-buffered LDS).
//
// Matrix-core layout (v_mfma_f32_16x16x32_bf16), as in the sparse kernel:
//   S^T  = K~ . Q~^T  A = 16 keys x 32 dims of K~, B = Q~^T (16 columns);
//   O^T += V^T . P^T  A = V^T (16 dims x 32 keys), B = P^T straight from the
//                     S^T registers (contraction index permuted to match).
// Softmax per column in fp32 with base-2 exponentials against a reference
// maximum fixed after the first key chunk (no rescaling of the 192 output
// accumulators, which live in AGPRs); a work-group whose logits outgrow that
// reference by more than 2^32 in probability redoes its walk exactly: the
// maximum over every key first, then the accumulation.
#include "qsa_common.h"
#include "attend_parts.h"

namespace qsa {

namespace {

constexpr int kDQ = 16;                 // queries per work-group
constexpr int kDKeys = 32;              // keys per chunk
constexpr int kDBlocks = kDKeys / kBlock;
constexpr int kDColTiles = 3;           // 48 columns per wave: 4 queries x 12 heads

// Two floats to a pair of bf16, round to nearest even (v_cvt_pk_bf16_f32),
// low half first; inputs are finite.
__device__ __forceinline__ uint32_t pk_bf16_hw(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

struct DenseBuf {
    u32x4 k[2 * 8 * 64];                // [key tile][k-step][lane]  16 KiB
    u32x4 v[16 * 64];                   // [dim tile][lane]          16 KiB
};

// Column c (0..47) of wave w: query 4w + c/12, head c%12 of the group.
__device__ __forceinline__ void dense_q_frags(const bf16_t *__restrict__ q, int64_t row /*token row of query 0 of
                                              the wave*/, int64_t pos /*its position*/, int grp, int ct,
                                              const Tables &tab, bf16x8 (&qf)[8])
{
    const int lane = threadIdx.x & 63;
    const int c = 16 * ct + (lane & 15);
    const int qi = c / kGroup, h = c % kGroup;
    const int g = lane >> 4;
    const bf16_t *src = q + ((row + qi) * kQHeads + grp * kGroup + h) * kHeadDim + 8 * g;
    u32x4 x[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] = *reinterpret_cast<const u32x4 *>(src + 32 * s);
    const int64_t p = pos + qi;
    const float *cs = tab.cos + p * kPairs + 8 * g;
    const float *sn = tab.sin + p * kPairs + 8 * g;
    uint32_t w0[4], w1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float r0[2], r1[2];
#pragma unroll
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
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = __builtin_bit_cast(bf16x8, x[s]);
}

// One chunk's K~ and V (8 blocks of one group, 2 KiB each) into registers.
// Thread t holds the 16-byte pieces x = t + 256 i (i = 0..3) of each: block
// blk0 + t/128 + 2i, bytes 16 (t%128) of it.  `edge` (the last chunk of a
// work-group's walk only): blocks past the caches' capacity are not read
// (zeros), and V of tokens after key position key_last is zeroed, so that the
// cache slots no query here may see (unwritten ones included) contribute
// exactly 0 to P.V whatever they hold.
__device__ __forceinline__ void dense_fetch(const char *__restrict__ kb, const char *__restrict__ vb, int64_t blk0,
                                            bool edge, int64_t nblk_cap, int64_t key_last, u32x4 (&pk)[4],
                                            u32x4 (&pv)[4])
{
    const int tid = static_cast<int>(threadIdx.x);
    const int64_t b0 = blk0 + (tid >> 7);
    const char *kp = kb + b0 * 2048 + 16 * (tid & 127);
    const char *vp = vb + b0 * 2048 + 16 * (tid & 127);
    if (!edge) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pk[i] = *reinterpret_cast<const u32x4 *>(kp + 4096 * i);
            pv[i] = *reinterpret_cast<const u32x4 *>(vp + 4096 * i);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t blk = b0 + 2 * i;
        const bool in = blk < nblk_cap;
        pk[i] = in ? *reinterpret_cast<const u32x4 *>(kp + 4096 * i) : u32x4{0u, 0u, 0u, 0u};
        u32x4 v = in ? *reinterpret_cast<const u32x4 *>(vp + 4096 * i) : u32x4{0u, 0u, 0u, 0u};
        // words {0,2} hold tokens 0|1 of the piece's two dims, {1,3} tokens 2|3
        const int64_t n_ok = key_last - blk * kBlock + 1;         // tokens 0 .. n_ok-1 are kept
        const uint32_t m01 = n_ok >= 2 ? 0xFFFFFFFFu : (n_ok == 1 ? 0x0000FFFFu : 0u);
        const uint32_t m23 = n_ok >= 4 ? 0xFFFFFFFFu : (n_ok == 3 ? 0x0000FFFFu : 0u);
        pv[i] = u32x4{v[0] & m01, v[1] & m23, v[2] & m01, v[3] & m23};
    }
}

// The pieces into LDS in operand order.  K~ piece x (block j = x/128; within
// the block dim group dg, token t, 8-dim part u) is row r = 4 (j%4) + t of key
// tile j/4, k-step dg, k-group u.  V piece x (block j, dims 2m, 2m+1, 4 tokens
// each) holds, for each of its two dims d, the 8 bytes that lane (d%16, j%4)
// of dim tile d/16 takes as k-elements 0..3 (j < 4) or 4..7 (j >= 4).  With
// j = t/128 + 2i both come to one per-thread base plus a constant per i.
__device__ __forceinline__ void dense_put(DenseBuf &buf, const u32x4 (&pk)[4], const u32x4 (&pv)[4])
{
    const int tid = static_cast<int>(threadIdx.x);
    const int h = tid >> 7, w = tid & 127;
    // K~: slot ((j/4) 8 + dg) 64 + 4 (j%4) + t + 16 u, j%4 = h + 2 (i%2), j/4 = i/2
    u32x4 *kdst = &buf.k[(w >> 4) * 64 + 4 * h + ((w >> 2) & 3) + 16 * (w & 3)];
    // V: dim d = 2w + e -> slot (d/16) 64 + d%16 + 16 (j%4), 8-byte half j/4
    u32x2 *vdst = reinterpret_cast<u32x2 *>(&buf.v[(w >> 3) * 64 + 2 * (w & 7) + 16 * h]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        kdst[(i >> 1) * 512 + 8 * (i & 1)] = pk[i];
        vdst[2 * (32 * (i & 1)) + (i >> 1)] = u32x2{pv[i][0], pv[i][1]};
        vdst[2 * (32 * (i & 1) + 1) + (i >> 1)] = u32x2{pv[i][2], pv[i][3]};
    }
}

}  // namespace

// Walk modes.  kStale: the reference maximum of each column is its maximum
// over the first chunk (keys 0..31, which every query sees); later logits may
// exceed it by up to kHeadroom (log2 units), so probabilities stay below
// 2^kHeadroom and nothing is rescaled; a column that would exceed the headroom
// raises the work-group's redo flag.  kMaxOnly: the exact maximum over all of
// a column's keys (logits only).  kFixed: accumulate with that exact maximum.
enum DenseMode { kStale = 0, kMaxOnly = 1, kFixed = 2 };
constexpr float kHeadroom = 32.0f;

struct DenseWave {
    bf16x8 qf[kDColTiles][8];           // Q~^T fragments of the wave's 48 columns
    int64_t qpos[kDColTiles];           // position of this lane's column's query, per column tile
    float m[kDColTiles], l[kDColTiles];
    f32x4 o[16][kDColTiles];            // O^T: dims 16n + 4g + j of this lane's column
};

template <int MODE>
__device__ __forceinline__ bool dense_walk(DenseBuf (&lds)[2], DenseWave &w, const bf16_t *__restrict__ kc,
                                           const bf16_t *__restrict__ vc, int nchunks, int64_t nblk_cap,
                                           int64_t p_first, int64_t p_last, float c2)
{
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    bool redo = false;
#pragma unroll
    for (int ct = 0; ct < kDColTiles; ++ct) {
        if (MODE != kFixed) w.m[ct] = -INFINITY;
        w.l[ct] = 0.f;
#pragma unroll
        for (int n = 0; n < 16; ++n) w.o[n][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    u32x4 pk[4], pv[4];
    const char *kb = reinterpret_cast<const char *>(kc), *vb = reinterpret_cast<const char *>(vc);
    dense_fetch(kb, vb, 0, nchunks == 1, nblk_cap, p_last, pk, pv);
    dense_put(lds[0], pk, pv);
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
        const DenseBuf &cur = lds[c & 1];
        const bool more = c + 1 < nchunks;
        if (more)
            dense_fetch(kb, vb, static_cast<int64_t>(c + 1) * kDBlocks, c + 2 == nchunks, nblk_cap, p_last, pk, pv);
        const int64_t k0 = static_cast<int64_t>(c) * kDKeys;
        const bool diag = k0 + kDKeys - 1 > p_first;         // some key may follow some query
        // ---- S^T for the chunk's two key tiles and the wave's three column tiles:
        // each K~ fragment is read from LDS once and feeds the three tiles.
        // Lane holds keys 16t + 4g + j of its column in sc[t][ct][j].
        f32x4 sc[2][kDColTiles];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int ct = 0; ct < kDColTiles; ++ct) sc[t][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const bf16x8 kf = __builtin_bit_cast(bf16x8, cur.k[(t * 8 + s) * 64 + lane]);
#pragma unroll
                for (int ct = 0; ct < kDColTiles; ++ct)
                    sc[t][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, w.qf[ct][s], sc[t][ct], 0, 0, 0);
            }
        }
        bf16x8 pf[kDColTiles];
        if (diag) {   // keys past a column's query get -inf (only the last chunk of a tile)
#pragma unroll
            for (int ct = 0; ct < kDColTiles; ++ct) {
                const int lim = static_cast<int>(w.qpos[ct] - k0) - 4 * g;      // key 16t + 4g + j kept iff 16t + j <= lim
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (16 * t + j > lim) sc[t][ct][j] = -INFINITY;
            }
        }
#pragma unroll
        for (int ct = 0; ct < kDColTiles; ++ct) {
            float cmax = fmaxf(fmaxf(fmaxf(sc[0][ct][0], sc[0][ct][1]), fmaxf(sc[0][ct][2], sc[0][ct][3])),
                               fmaxf(fmaxf(sc[1][ct][0], sc[1][ct][1]), fmaxf(sc[1][ct][2], sc[1][ct][3])));
            cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
            cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
            if (MODE == kMaxOnly) {
                w.m[ct] = fmaxf(w.m[ct], cmax);
                continue;
            }
            if (MODE == kStale) {
                if (c == 0) w.m[ct] = cmax;
                else redo |= (cmax - w.m[ct]) * c2 > kHeadroom;
            }
            const float mc = w.m[ct] * c2;
            uint32_t pw[4];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                float p[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(sc[t][ct][j] * c2 - mc);
                pw[2 * t] = pk_bf16_hw(p[0], p[1]);
                pw[2 * t + 1] = pk_bf16_hw(p[2], p[3]);
            }
            // the denominator sums the bf16 probabilities the PV product uses
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                psum += __uint_as_float(pw[i] << 16) + __uint_as_float(pw[i] & 0xFFFF0000u);
            w.l[ct] += psum;
            pf[ct] = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
        }
        if (MODE != kMaxOnly) {
            // ---- O^T += V^T . P^T: each V fragment is read once and feeds the three tiles
#pragma unroll
            for (int n = 0; n < 16; ++n) {
                const bf16x8 vf = __builtin_bit_cast(bf16x8, cur.v[n * 64 + lane]);
#pragma unroll
                for (int ct = 0; ct < kDColTiles; ++ct)
                    w.o[n][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[ct], w.o[n][ct], 0, 0, 0);
            }
        }
        // the other buffer was last read in chunk c - 1, before the barrier that ended it
        if (more) dense_put(lds[(c + 1) & 1], pk, pv);
        __syncthreads();
    }
    return redo;
}

// out rows row0 .. row0+L-1 of buffers holding ld rows per sequence, at query
// positions q_offset + row; keys 0 .. position from the caches.
__global__ __launch_bounds__(256, 1) void dense_attend_kernel(
    Tables tab, int64_t L, int64_t row0, int64_t ld, int64_t q_offset, int64_t nblk_cap, float c2,
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k_cache, const bf16_t *__restrict__ v_cache,
    bf16_t *__restrict__ out)
{
    __shared__ DenseBuf lds[2];
    __shared__ int redo_any;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, g = lane >> 4;
    const int64_t b = blockIdx.y;
    const int grp = static_cast<int>(blockIdx.z);
    const int64_t ntile = (L + kDQ - 1) / kDQ;
    const int64_t tile = ntile - 1 - static_cast<int64_t>(blockIdx.x);          // longest rows first
    const int64_t i0 = tile * kDQ;                                                 // first query of the tile
    const int64_t last = (i0 + kDQ < L ? i0 + kDQ : L) - 1;
    const int64_t p_first = q_offset + row0 + i0;
    const int64_t p_last = q_offset + row0 + last;
    const int nchunks = static_cast<int>(p_last / kDKeys) + 1;
    if (threadIdx.x == 0) redo_any = 0;

    // this wave's queries (clamped into the call's rows; clamped ones are not stored)
    const int64_t iw = i0 + 4 * wave;
    const int64_t iw_c = iw < L ? iw : L - 1;
    const int nq = static_cast<int>(iw < L ? (L - iw < 4 ? L - iw : 4) : 0);
    DenseWave w;
#pragma unroll
    for (int ct = 0; ct < kDColTiles; ++ct) {
        const int qi = (16 * ct + col) / kGroup;
        const int64_t r = (iw_c + qi < L) ? iw_c : iw_c - qi;      // keep the loads inside the call's rows
        dense_q_frags(q + (b * ld + row0) * kQHeads * kHeadDim, r, q_offset + row0 + r, grp, ct, tab, w.qf[ct]);
        w.qpos[ct] = q_offset + row0 + r + qi;
    }
    const bf16_t *kc = k_cache + kcache_block_base(b, grp, 0, nblk_cap);
    const bf16_t *vc = v_cache + kcache_block_base(b, grp, 0, nblk_cap);

    const bool redo = dense_walk<kStale>(lds, w, kc, vc, nchunks, nblk_cap, p_first, p_last, c2);
    if (__builtin_amdgcn_ballot_w64(redo) && lane == 0) atomicOr(&redo_any, 1);
    __syncthreads();
    if (redo_any) {        // rare: some logit beyond the headroom -- exact maximum first, then accumulate
        dense_walk<kMaxOnly>(lds, w, kc, vc, nchunks, nblk_cap, p_first, p_last, c2);
        dense_walk<kFixed>(lds, w, kc, vc, nchunks, nblk_cap, p_first, p_last, c2);
    }

    // ---- normalise and store: lane holds dims 16n + 4g + j of its column
#pragma unroll
    for (int ct = 0; ct < kDColTiles; ++ct) {
        float lt = w.l[ct] + __shfl_xor(w.l[ct], 16);
        lt += __shfl_xor(lt, 32);
        const float inv = 1.0f / lt;
        const int cc = 16 * ct + col;
        const int qi = cc / kGroup, h = cc % kGroup;
        if (qi >= nq) continue;
        bf16_t *dst = out + ((b * ld + row0 + iw + qi) * kQHeads + grp * kGroup + h) * kHeadDim + 4 * g;
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            const u32x2 v = u32x2{pack_bf16x2(w.o[n][ct][0] * inv, w.o[n][ct][1] * inv),
                                  pack_bf16x2(w.o[n][ct][2] * inv, w.o[n][ct][3] * inv)};
            *reinterpret_cast<u32x2 *>(dst + 16 * n) = v;
        }
    }
}

hipError_t launch_dense_attend(const Tables &tab, hipStream_t st, int32_t B, int64_t L, int64_t row0, int64_t ld,
                               int64_t q_offset, int64_t nblk_cap, float sigma, const bf16_t *q,
                               const bf16_t *k_cache, const bf16_t *v_cache, bf16_t *out)
{
    if (L <= 0 || B <= 0) return hipSuccess;
    const int64_t ntile = (L + kDQ - 1) / kDQ;
    dim3 grid(static_cast<unsigned>(ntile), static_cast<unsigned>(B), static_cast<unsigned>(kKVHeads));
    hipLaunchKernelGGL(dense_attend_kernel, grid, dim3(256), 0, st, tab, L, row0, ld, q_offset, nblk_cap,
                       sigma * kLog2e, q, k_cache, v_cache, out);
    return hipGetLastError();
}

}  // namespace qsa
