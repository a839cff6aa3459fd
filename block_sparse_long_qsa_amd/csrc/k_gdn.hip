// Gated DeltaNet chunked prefill (PyTorchKR post "Qwen3.8-Flash-Next, 1/9의
// 학습 비용으로 …", section "어텐션: GDN이 기억하고 QSA가 찾아낸다": the gated
// delta rule S_t = (alpha_t I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T;
// spec table: 48 V heads, 16 QK heads, head dim 128; section "FlashQLA": the
// chunked-prefill call takes q, k [T, H_q, 128], v [T, H_v, 128], the log gate
// g and beta [T, H_v], a scale, an optional initial state [H_v, 128, 128],
// returns the final state, and packs variable-length sequences by offsets).
//
// With u_t = beta_t (v_t - S_{t-1}^T k_t), the value the delta rule writes, the
// rule reads S_t = alpha_t S_{t-1} + k_t u_t^T.  Inside a chunk of C = 64 tokens
// entered with state S_0, let G_t be the inclusive prefix sum of g = ln alpha
// and gamma_t = exp(G_t).  Unrolling S_{t-1} gives a unit lower-triangular
// system for the rows of U:
//   (I + Lt) U = diag(beta) X,   X = V - diag(gamma_{t-1}) K S_0,
//   Lt[t][j] = beta_t exp(G_{t-1} - G_j) k_t.k_j            (j < t),
// so U = Tb X with Tb = (I + Lt)^{-1} diag(beta), and
//   O   = diag(scale gamma_t) Q S_0 + P U,  P[t][j] = scale exp(G_t - G_j) q_t.k_j  (j <= t),
//   S_C = gamma_C S_0 + K^T diag(exp(G_C - G_t)) U.
// Tb and P do not depend on the state: gdn_prep_kernel builds them for every
// (chunk, V head) in parallel, together with K^T of every (chunk, QK head).
// gdn_scan_kernel then walks the chunks of one (sequence, V head, 16*NW value
// columns) in order with its columns of S in registers (each column of S
// evolves on its own), so a head's state is advanced by 128/(16*NW)
// work-groups at once; its memory traffic runs on separate producer and store
// waves (see gdn_scan_kernel).
//
// Matrix cores: v_mfma_f32_16x16x32_bf16; A lane l = row l%16, k = 8(l/16)..+7;
// B lane l = column l%16, same k; C lane l = rows 4(l/16)..+3, column l%16.
// Accumulator tiles that feed a later product as its B operand (S, X, U) are
// rounded to bf16 and passed through a small per-wave LDS transpose.
//
// Tile layout (LDS and workspace alike): rows of 16-byte chunks, chunk c of
// row r stored at position c ^ (r & 15) in 256-byte rows (128 bf16 wide) and
// c ^ ((r >> 1) & 7) in 128-byte rows (64 wide), so that the 16 rows a
// fragment read touches fall in distinct LDS banks.
#include "qsa_common.h"

namespace qsa {

constexpr int kGdnDim = 128;     // q/k/v head dim
constexpr int kGdnChunk = 64;    // tokens per chunk
constexpr int kGdnPad = 136;     // LDS row stride (bf16) of 128-wide tiles
constexpr int kGdnPad64 = 72;    // LDS row stride (bf16) of 64-wide tiles
constexpr int kGdnTile = kGdnChunk * kGdnChunk;   // one 64 x 64 matrix of the workspace

// Tokens [base, base + len) of sequence s.  Offsets are clamped to the packed
// token range and the length to max_len, so no offset table can address memory
// outside q/k/v/o or the workspace.
struct GdnSpan {
    int64_t base;
    int len;
};
__device__ __forceinline__ GdnSpan gdn_span(const int32_t *__restrict__ cu, int s, int64_t n_tok, int max_len) {
    int64_t a = cu[s], b = cu[s + 1];
    a = a < 0 ? 0 : (a > n_tok ? n_tok : a);
    b = b < a ? a : (b > n_tok ? n_tok : b);
    if (b - a > max_len) b = a + max_len;
    return {a, static_cast<int>(b - a)};
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_prefix_sum(float x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    return x;
}

__device__ __forceinline__ f32x4 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Workspace: for every (sequence, V head, chunk) Tb then P, [64][64] bf16 each
// (16 KiB); after all of them, for every (sequence, QK head, chunk) K^T
// [128][64] bf16 (16 KiB).  Offsets in bf16 elements.
__device__ __forceinline__ int64_t gdn_ws_off(int s, int hv, int Hv, int nchunk_cap, int c) {
    return ((static_cast<int64_t>(s) * Hv + hv) * nchunk_cap + c) * (2 * kGdnTile);
}
__device__ __forceinline__ int64_t gdn_kt_off(int nseq, int s, int hq, int Hq, int Hv, int nchunk_cap, int c) {
    return static_cast<int64_t>(nseq) * Hv * nchunk_cap * (2 * kGdnTile) +
           ((static_cast<int64_t>(s) * Hq + hq) * nchunk_cap + c) * (2 * kGdnTile);
}

// Byte offset of 16-byte chunk cc of row r in a swizzled tile.
__device__ __forceinline__ int sw128(int r, int cc) { return r * 256 + ((cc ^ (r & 15)) << 4); }
__device__ __forceinline__ int sw64(int r, int cc) { return r * 128 + ((cc ^ ((r >> 1) & 7)) << 4); }

__device__ __forceinline__ float exp_e(float x) { return exp2f(x * 1.4426950408889634f); }

// Two floats to a pair of bf16 (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Barriers that order LDS only: global stores and loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// A barrier with no memory fence (the caller has waited for what it needs);
// the empty asm statements keep the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void raw_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void lds_wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (and nothing else).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Renumber work-group ids so that consecutive logical ids run on one XCD
// (work-groups are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ int64_t xcd_local_id() {
    const int64_t n = gridDim.x, b = blockIdx.x;
    return n % 8 == 0 ? (b % 8) * (n / 8) + b / 8 : b;
}

// ---------------------------------------------------------------------------
// One wave per (sequence, chunk, V head): K K^T and Q K^T of the chunk (the 10
// causal 16 x 16 tiles) on the matrix cores from fragments read straight from
// q and k; Lt into LDS and P to the workspace; Tb by forward substitution, one
// column per lane.  The first V head of each QK head also writes K^T.  Rows
// past the end of the sequence repeat its last token: their beta is 0, so
// their rows of Lt and Tb are zero (and so is every Tb column they own), and
// causality zeroes their P columns for every real row.
__global__ __launch_bounds__(64) void gdn_prep_kernel(const int32_t *__restrict__ cu, int64_t n_tok, int max_len,
                                                      int nchunk_cap, int nseq, int Hq, int Hv, float scale,
                                                      const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
                                                      const float *__restrict__ g, const float *__restrict__ beta,
                                                      bf16_t *__restrict__ ws)
{
    __shared__ __align__(16) float Lt[kGdnTile];    // 16 KiB; first the K^T staging tile
    __shared__ float sG[kGdnChunk], sB[kGdnChunk];

    const int64_t e = xcd_local_id();
    const int hv = static_cast<int>(e % Hv);
    const int c = static_cast<int>((e / Hv) % nchunk_cap);
    const int s = static_cast<int>(e / (static_cast<int64_t>(Hv) * nchunk_cap));
    const GdnSpan sp = gdn_span(cu, s, n_tok, max_len);
    const int t0 = c * kGdnChunk;
    if (t0 >= sp.len) return;
    const int nt = min(kGdnChunk, sp.len - t0), last = nt - 1;
    const int rep = Hv / Hq, hq = hv / rep;
    const int lane = threadIdx.x, lr = lane & 15, lg = lane >> 4;
    const int64_t tok0 = sp.base + t0;
    const int kstride = Hq * kGdnDim;

    bf16x8 kf[4][4], qf[4][4];   // rows 16i + l%16, dims 32s + 8(l/16) ..
    {
        const bf16_t *kb = k + (tok0 * Hq + hq) * kGdnDim + 8 * lg;
        const bf16_t *qb = q + (tok0 * Hq + hq) * kGdnDim + 8 * lg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = min(16 * i + lr, last);
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                kf[i][s4] = *reinterpret_cast<const bf16x8 *>(kb + row * kstride + 32 * s4);
                qf[i][s4] = *reinterpret_cast<const bf16x8 *>(qb + row * kstride + 32 * s4);
            }
        }
    }
    {
        const int64_t gi = (tok0 + min(lane, last)) * Hv + hv;
        const float gv = g[gi], bv = beta[gi];
        sG[lane] = wave_prefix_sum(lane < nt ? gv : 0.f);
        sB[lane] = lane < nt ? bv : 0.f;
    }
    f32x4 kk[10], qk[10];   // tile (w, jt), jt <= w, at index w(w+1)/2 + jt
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int jt = 0; jt <= w; ++jt) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                a = mfma32(kf[w][s4], kf[jt][s4], a);
                b = mfma32(qf[w][s4], kf[jt][s4], b);
            }
            kk[w * (w + 1) / 2 + jt] = a;
            qk[w * (w + 1) / 2 + jt] = b;
        }

    if (hv % rep == 0) {
        // K^T of the chunk, through LDS: element (dim d, token t) at sw64(d, t/8) + 2(t%8).
        unsigned char *tk = reinterpret_cast<unsigned char *>(Lt);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const u32x4 w4 = __builtin_bit_cast(u32x4, kf[i][s4]);
                const int t = 16 * i + lr;
#pragma unroll
                for (int e8 = 0; e8 < 8; ++e8) {
                    const int d = 32 * s4 + 8 * lg + e8;
                    const uint32_t word = w4[e8 >> 1];
                    *reinterpret_cast<bf16_t *>(tk + sw64(d, t >> 3) + 2 * (t & 7)) =
                        static_cast<bf16_t>((e8 & 1) ? (word >> 16) : (word & 0xFFFFu));
                }
            }
        wave_sync();
        bf16_t *kt = ws + gdn_kt_off(nseq, s, hq, Hq, Hv, nchunk_cap, c);
#pragma unroll
        for (int m = 0; m < 16; ++m)
            *reinterpret_cast<u32x4 *>(kt + 8 * (lane + 64 * m)) = *reinterpret_cast<const u32x4 *>(tk + 16 * (lane + 64 * m));
        wave_sync();
    }
    wave_sync();

    bf16_t *Tb = ws + gdn_ws_off(s, hv, Hv, nchunk_cap, c);
    unsigned char *P = reinterpret_cast<unsigned char *>(Tb + kGdnTile);
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * w + 4 * lg + j, jj = 16 * jt + lr;
                float pv = 0.f;
                if (jt <= w) {
                    const float Gj = sG[jj];
                    const float Gprev = t > 0 ? sG[t - 1] : 0.f;
                    const float lv = jj < t ? sB[t] * exp_e(Gprev - Gj) * kk[w * (w + 1) / 2 + jt][j] : 0.f;
                    if (jj <= t) pv = scale * exp_e(sG[t] - Gj) * qk[w * (w + 1) / 2 + jt][j];
                    Lt[t * kGdnChunk + jj] = lv;   // tiles right of the diagonal are never read
                }
                *reinterpret_cast<bf16_t *>(P + sw64(t, jj >> 3) + 2 * (jj & 7)) = f32_to_bf16(pv);
            }
    wave_sync();

    // Column `lane` of T = (I + Lt)^{-1}: x_t = [t == lane] - sum_{j<t} Lt[t][j] x_j.
    // x_j is still zero for j >= t and so is Lt[t][j]: whole float4 reads are exact.
    float x[kGdnChunk];
#pragma unroll
    for (int t = 0; t < kGdnChunk; ++t) x[t] = 0.f;
    x[0] = lane == 0 ? 1.f : 0.f;
#pragma unroll
    for (int t = 1; t < kGdnChunk; ++t) {
        f32x4 row[kGdnChunk / 4];
#pragma unroll
        for (int j4 = 0; j4 < (t + 3) / 4; ++j4) row[j4] = *reinterpret_cast<const f32x4 *>(Lt + t * kGdnChunk + 4 * j4);
        float a0 = lane == t ? 1.f : 0.f, a1 = 0.f;
#pragma unroll
        for (int j4 = 0; j4 < (t + 3) / 4; ++j4) {
            a0 = fmaf(-row[j4][0], x[4 * j4 + 0], a0);
            a1 = fmaf(-row[j4][1], x[4 * j4 + 1], a1);
            a0 = fmaf(-row[j4][2], x[4 * j4 + 2], a0);
            a1 = fmaf(-row[j4][3], x[4 * j4 + 3], a1);
        }
        x[t] = a0 + a1;
    }
    const float bc = sB[lane];
    unsigned char *tb = reinterpret_cast<unsigned char *>(Tb);
#pragma unroll
    for (int t = 0; t < kGdnChunk; ++t)
        *reinterpret_cast<bf16_t *>(tb + sw64(t, lane >> 3) + 2 * (lane & 7)) = f32_to_bf16(x[t] * bc);
}

// ---------------------------------------------------------------------------
// Chunk walk of one (sequence, V head, 16*NW value columns).  Compute wave w
// owns the 16 columns c0 = 16*(NW*slice + w) .. +15 of S (rows 16i + 4(l/16)
// + j of column c0 + l%16 in S[i][j]).  Per chunk, from LDS only:
//   R_K = K S, R_Q = Q S                                  (32 products)
//   X = V - diag(gamma_{t-1}) R_K;  U = Tb X              (8)
//   O = diag(scale gamma_t) R_Q + P U                     (8)
//   S = gamma_C S + K^T diag(exp(G_C - G_t)) U            (16)
// All global traffic of the walk runs on other waves, so a compute wave never
// waits on memory: two producer waves copy each chunk's tiles into a two-slot
// LDS ring with the LDS-DMA path (global_load_lds), and a store wave writes
// each chunk's O from LDS while the next chunk computes.  Each chunk step has
// two barriers: A after the products with K and Q, B at the end.  A slot's K, Q
// part is refilled (two chunks ahead) as soon as barrier A releases it and its
// other part (K^T, Tb, P, V) after barrier B, so every copy has more than one
// step to land: K, Q of chunk c+1 must be in by barrier B of chunk c, the rest
// by barrier A of chunk c+1.
template <int NW>
__global__ __launch_bounds__(64 * (NW + 3)) void gdn_scan_kernel(
    const int32_t *__restrict__ cu, int64_t n_tok, int max_len, int nchunk_cap, int nseq, int Hq, int Hv, float scale,
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k, const bf16_t *__restrict__ v,
    const float *__restrict__ g, const bf16_t *__restrict__ ws, const float *s0, bf16_t *__restrict__ o, float *s_out)
{
    constexpr int kCols = 16 * NW;                    // value columns of the work-group
    constexpr int kSlices = kGdnDim / kCols;
    // One ring slot: K, Q (sw128), K^T, Tb, P (sw64), V [64][kCols] bf16.
    constexpr int oQ = 16384, oKt = 32768, oTb = 49152, oP = 57344, oV = 65536;
    constexpr int kSlot = oV + kGdnChunk * kCols * 2;
    constexpr int kVPieces = (kSlot - oV) / 1024;
    constexpr int kE = 4 * kGdnChunk;                 // exp(G_{t-1}), scale exp(G_t), exp(G_C - G_t), exp(G_C)
    static_assert(kSlot % 1024 == 0, "ring slot must be whole 1 KiB pieces");
    __shared__ __align__(16) unsigned char sbuf[2 * kSlot];
    __shared__ __align__(16) float sg[3][kGdnChunk];            // gates g, three chunks
    __shared__ __align__(16) bf16_t sO[2][kGdnChunk * kCols];   // O staging, [token][kCols]
    __shared__ __align__(16) bf16_t sTr[NW][16 * kGdnPad];
    __shared__ __align__(16) float sE[2 * kE];

    const int64_t e = xcd_local_id();
    const int slice = static_cast<int>(e % kSlices);
    const int hv = static_cast<int>((e / kSlices) % Hv);
    const int s = static_cast<int>(e / (static_cast<int64_t>(kSlices) * Hv));
    const int hq = hv / (Hv / Hq);

    // The wave index is read into a scalar register: the roles below branch on it
    // and the LDS-DMA destination (M0) is computed from it.
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const GdnSpan sp = gdn_span(cu, s, n_tok, max_len);
    const int nck = (sp.len + kGdnChunk - 1) / kGdnChunk;
    const int kstride = Hq * kGdnDim, vstride = Hv * kGdnDim;
    const int col0 = kCols * slice;                   // first value column of the work-group

    auto chunk_nt = [&](int c) { return min(kGdnChunk, sp.len - c * kGdnChunk); };

    // ---- producer waves.  Group KQ of chunk c: producer 0 copies K, producer 1
    // copies Q and the gates (into sg[c % 3]); group TPKV: producer 0 copies Tb,
    // P and the V columns, producer 1 copies K^T.  Rows past the end of the
    // sequence repeat its last token (see gdn_prep_kernel for why that is
    // harmless).  Issue order per producer: ..., KQ(c+1) [after A(c-1)],
    // TPKV(c+1) [after B(c-1)], KQ(c+2) [after A(c)], ...; so before A(c)
    // (TPKV(c) landed) and before B(c) (KQ(c+1) landed) the wave may leave the
    // two younger groups in flight.
    if (w > NW) {
        const int pw = w - NW - 1;
        const int lrow = lane >> 4, lcp = lane & 15, rowbytes = kstride * 2;
        auto slot = [&](int c) { return sbuf + (c & 1) * kSlot; };
        auto copy_kq = [&](int c) {
            unsigned char *dst = slot(c);
            const int last = chunk_nt(c) - 1;
            const int64_t tok0 = sp.base + c * kGdnChunk;
            const unsigned char *rows = reinterpret_cast<const unsigned char *>((pw == 0 ? k : q) + (tok0 * Hq + hq) * kGdnDim);
            unsigned char *drows = dst + (pw == 0 ? 0 : oQ);
#pragma unroll
            for (int n = 0; n < 16; ++n) {         // rows 4n .. 4n+3, swizzled 16-byte chunks
                const int row = 4 * n + lrow;
                const int src = min(row, last) * rowbytes + 16 * (lcp ^ ((4 * (n & 3)) + lrow));
                __builtin_amdgcn_global_load_lds(rows + src, drows + 1024 * n, 16, 0, 0);
            }
            if (pw == 1)
                __builtin_amdgcn_global_load_lds(g + (tok0 + min(lane, last)) * Hv + hv, static_cast<void *>(sg[c % 3]), 4, 0, 0);
        };
        auto copy_tpkv = [&](int c) {
            unsigned char *dst = slot(c);
            const int last = chunk_nt(c) - 1;
            const int64_t tok0 = sp.base + c * kGdnChunk;
            const unsigned char *flat = reinterpret_cast<const unsigned char *>(
                pw == 0 ? ws + gdn_ws_off(s, hv, Hv, nchunk_cap, c) : ws + gdn_kt_off(nseq, s, hq, Hq, Hv, nchunk_cap, c));
            unsigned char *dflat = dst + (pw == 0 ? oTb : oKt);
#pragma unroll
            for (int n = 0; n < 16; ++n)           // Tb then P, or K^T: contiguous 16 KiB
                __builtin_amdgcn_global_load_lds(flat + 1024 * n + 16 * lane, dflat + 1024 * n, 16, 0, 0);
            if (pw == 0) {
                constexpr int kChunksPerRow = kCols / 8;
                constexpr int kRowsPerPiece = 64 / kChunksPerRow;
                const unsigned char *vr = reinterpret_cast<const unsigned char *>(v + (tok0 * Hv + hv) * kGdnDim + col0);
#pragma unroll
                for (int n = 0; n < kVPieces; ++n) {
                    const int row = n * kRowsPerPiece + lane / kChunksPerRow;
                    const int64_t src = static_cast<int64_t>(min(row, last)) * vstride * 2 + 16 * (lane % kChunksPerRow);
                    __builtin_amdgcn_global_load_lds(vr + src, dst + oV + 1024 * n, 16, 0, 0);
                }
            }
        };
        // vmcnt immediates: n_KQ + n_TPKV, n_KQ, n_TPKV (per producer), and 0.
        auto wait_groups = [&](bool kq, bool tpkv) {
            if (pw == 0) {
                if (kq && tpkv) __builtin_amdgcn_s_waitcnt(vmcnt_imm(16 + 16 + kVPieces));
                else if (kq) __builtin_amdgcn_s_waitcnt(vmcnt_imm(16));
                else if (tpkv) __builtin_amdgcn_s_waitcnt(vmcnt_imm(16 + kVPieces));
                else __builtin_amdgcn_s_waitcnt(0);
            } else {
                if (kq && tpkv) __builtin_amdgcn_s_waitcnt(vmcnt_imm(17 + 16));
                else if (kq) __builtin_amdgcn_s_waitcnt(vmcnt_imm(17));
                else if (tpkv) __builtin_amdgcn_s_waitcnt(vmcnt_imm(16));
                else __builtin_amdgcn_s_waitcnt(0);
            }
        };
        if (nck > 0) {
            copy_kq(0);
            copy_tpkv(0);
        }
        if (nck > 1) copy_kq(1);
        wait_groups(nck > 1, false);                  // chunk 0 whole
        raw_barrier();                                // B(-1)
        for (int c = 0; c < nck; ++c) {
            if (c + 1 < nck) copy_tpkv(c + 1);
            wait_groups(c + 1 < nck, c + 1 < nck);    // TPKV(c)
            raw_barrier();                            // A(c)
            if (c + 2 < nck) copy_kq(c + 2);
            wait_groups(c + 2 < nck, c + 1 < nck);    // KQ(c+1)
            raw_barrier();                            // B(c)
        }
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }

    // ---- store wave: O of chunk c-1 from sO[(c-1)&1] while chunk c computes.
    if (w == NW) {
        constexpr int kChunksPerRow = kCols / 8;
        auto store = [&](int c) {
            const int nt = chunk_nt(c);
            const bf16_t *src = sO[c & 1];
#pragma unroll
            for (int n = 0; n < kGdnChunk * kChunksPerRow / 64; ++n) {
                const int idx = lane + 64 * n, t = idx / kChunksPerRow, cc = idx % kChunksPerRow;
                const u32x4 val = *reinterpret_cast<const u32x4 *>(src + t * kCols + 8 * cc);
                if (t < nt)
                    *reinterpret_cast<u32x4 *>(o + ((sp.base + c * kGdnChunk + t) * Hv + hv) * kGdnDim + col0 + 8 * cc) = val;
            }
        };
        lds_barrier();                                // B(-1)
        for (int c = 0; c < nck; ++c) {
            if (c > 0) store(c - 1);
            lds_barrier();                            // A(c)
            lds_barrier();                            // B(c)
        }
        if (nck > 0) store(nck - 1);
        return;
    }

    // ---- compute waves
    const int lcol = 16 * w + lr;                     // column within the work-group
    const int col = col0 + lcol;
    const int64_t sbase = (static_cast<int64_t>(s) * Hv + hv) * kGdnDim * kGdnDim;
    f32x4 S[8];
    if (s0) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[i][j] = s0[sbase + (16 * i + 4 * lg + j) * kGdnDim + col];
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    auto gates = [&](int c, float *ed) {              // wave 0
        const float G = wave_prefix_sum(lane < chunk_nt(c) ? sg[c % 3][lane] : 0.f);
        const float Gprev = __shfl_up(G, 1);
        const float GC = __shfl(G, 63);
        ed[lane] = lane == 0 ? 1.f : exp_e(Gprev);
        ed[kGdnChunk + lane] = scale * exp_e(G);
        ed[2 * kGdnChunk + lane] = exp_e(GC - G);
        ed[3 * kGdnChunk + lane] = exp_e(GC);
    };
    bf16_t *tr = sTr[w];

    lds_barrier();                                    // B(-1): chunk 0 and the gates of chunk 0 have landed
    for (int c = 0; c < nck; ++c) {
        const unsigned char *cur = sbuf + (c & 1) * kSlot;
        const unsigned char *bK = cur, *bQ = cur + oQ, *bKt = cur + oKt, *bTb = cur + oTb, *bP = cur + oP;
        const bf16_t *bV = reinterpret_cast<const bf16_t *>(cur + oV);
        float *ec = sE + (c & 1) * kE;
        if (w == 0) gates(c, ec);                     // read by every compute wave after barrier A

        // S -> bf16 B operand (k = rows of S).
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<u32x2 *>(tr + lr * kGdnPad + 16 * i + 4 * lg) =
                u32x2{pk_bf16(S[i][0], S[i][1]), pk_bf16(S[i][2], S[i][3])};
        bf16x8 ak[4][4], aq[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                ak[i][s4] = *reinterpret_cast<const bf16x8 *>(bK + sw128(16 * i + lr, 4 * s4 + lg));
                aq[i][s4] = *reinterpret_cast<const bf16x8 *>(bQ + sw128(16 * i + lr, 4 * s4 + lg));
            }
        lds_wave_sync();
        bf16x8 bs[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) bs[s4] = *reinterpret_cast<const bf16x8 *>(tr + lr * kGdnPad + 32 * s4 + 8 * lg);
        f32x4 rk[4], rq[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rk[i] = rq[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                rk[i] = mfma32(ak[i][s4], bs[s4], rk[i]);
                rq[i] = mfma32(aq[i][s4], bs[s4], rq[i]);
            }
        }
        lds_barrier();                                // A(c): K and Q of this slot are free
        bf16x8 atb[4][2], ap[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                atb[i][s2] = *reinterpret_cast<const bf16x8 *>(bTb + sw64(16 * i + lr, 4 * s2 + lg));
                ap[i][s2] = *reinterpret_cast<const bf16x8 *>(bP + sw64(16 * i + lr, 4 * s2 + lg));
            }
        f32x4 ep[4], eg[4], et[4];
        float vv[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ep[i] = *reinterpret_cast<const f32x4 *>(ec + 16 * i + 4 * lg);
            eg[i] = *reinterpret_cast<const f32x4 *>(ec + kGdnChunk + 16 * i + 4 * lg);
            et[i] = *reinterpret_cast<const f32x4 *>(ec + 2 * kGdnChunk + 16 * i + 4 * lg);
#pragma unroll
            for (int j = 0; j < 4; ++j) vv[4 * i + j] = bf16_to_f32(bV[(16 * i + 4 * lg + j) * kCols + lcol]);
        }
        const float gC = ec[3 * kGdnChunk];
        // X = V - diag(gamma_{t-1}) K S, rows = tokens.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float xv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) xv[j] = vv[4 * i + j] - ep[i][j] * rk[i][j];
            *reinterpret_cast<u32x2 *>(tr + lr * kGdnPad + 16 * i + 4 * lg) = u32x2{pk_bf16(xv[0], xv[1]), pk_bf16(xv[2], xv[3])};
        }
        lds_wave_sync();
        bf16x8 bx[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) bx[s2] = *reinterpret_cast<const bf16x8 *>(tr + lr * kGdnPad + 32 * s2 + 8 * lg);
        f32x4 U[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            U[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) U[i] = mfma32(atb[i][s2], bx[s2], U[i]);
        }
        bf16x8 akt[8][2];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) akt[i][s2] = *reinterpret_cast<const bf16x8 *>(bKt + sw64(16 * i + lr, 4 * s2 + lg));
        // U (for P U) in rows 0..63 and diag(exp(G_C - G_t)) U (for K^T) in rows 64..127.
        lds_wave_sync();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tb = 16 * i + 4 * lg;
            *reinterpret_cast<u32x2 *>(tr + lr * kGdnPad + tb) = u32x2{pk_bf16(U[i][0], U[i][1]), pk_bf16(U[i][2], U[i][3])};
            *reinterpret_cast<u32x2 *>(tr + lr * kGdnPad + 64 + tb) =
                u32x2{pk_bf16(et[i][0] * U[i][0], et[i][1] * U[i][1]), pk_bf16(et[i][2] * U[i][2], et[i][3] * U[i][3])};
        }
        lds_wave_sync();
        bf16x8 bu[2], bw[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            bu[s2] = *reinterpret_cast<const bf16x8 *>(tr + lr * kGdnPad + 32 * s2 + 8 * lg);
            bw[s2] = *reinterpret_cast<const bf16x8 *>(tr + lr * kGdnPad + 64 + 32 * s2 + 8 * lg);
        }
        // O = diag(scale gamma_t) Q S + P U, staged as bf16 for the store wave.
        bf16_t *so = sO[c & 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 acc;
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = eg[i][j] * rq[i][j];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) acc = mfma32(ap[i][s2], bu[s2], acc);
            const uint32_t p01 = pk_bf16(acc[0], acc[1]), p23 = pk_bf16(acc[2], acc[3]);
            const int tb = 16 * i + 4 * lg;
            so[(tb + 0) * kCols + lcol] = static_cast<bf16_t>(p01 & 0xFFFFu);
            so[(tb + 1) * kCols + lcol] = static_cast<bf16_t>(p01 >> 16);
            so[(tb + 2) * kCols + lcol] = static_cast<bf16_t>(p23 & 0xFFFFu);
            so[(tb + 3) * kCols + lcol] = static_cast<bf16_t>(p23 >> 16);
        }
        // S = gamma_C S + K^T diag(exp(G_C - G_t)) U
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) S[i][j] *= gC;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) S[i] = mfma32(akt[i][s2], bw[s2], S[i]);
        }
        lds_barrier();                                // B(c)
    }
    if (s_out) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) s_out[sbase + (16 * i + 4 * lg + j) * kGdnDim + col] = S[i][j];
    }
}

constexpr int kGdnScanWaves = 2;      // compute waves of a scan work-group (32 value columns)

hipError_t launch_gdn_prep(hipStream_t stream, int nseq, const int32_t *cu, int64_t n_tok, int max_len, int Hq, int Hv,
                           float scale, const bf16_t *q, const bf16_t *k, const float *g, const float *beta, bf16_t *ws)
{
    const int nchunk_cap = (max_len + kGdnChunk - 1) / kGdnChunk;
    if (nchunk_cap == 0) return hipSuccess;
    const int64_t nwg = static_cast<int64_t>(nseq) * nchunk_cap * Hv;
    hipLaunchKernelGGL(gdn_prep_kernel, dim3(static_cast<unsigned>(nwg)), dim3(64), 0, stream, cu, n_tok, max_len,
                       nchunk_cap, nseq, Hq, Hv, scale, q, k, g, beta, ws);
    return hipGetLastError();
}

hipError_t launch_gdn_scan(hipStream_t stream, int nseq, const int32_t *cu, int64_t n_tok, int max_len, int Hq, int Hv,
                           float scale, const bf16_t *q, const bf16_t *k, const bf16_t *v, const float *g,
                           const float *s0, bf16_t *o, float *s_out, const bf16_t *ws)
{
    const int nchunk_cap = (max_len + kGdnChunk - 1) / kGdnChunk;
    constexpr int kSlices = kGdnDim / (16 * kGdnScanWaves);
    const int64_t nwg = static_cast<int64_t>(nseq) * Hv * kSlices;
    hipLaunchKernelGGL((gdn_scan_kernel<kGdnScanWaves>), dim3(static_cast<unsigned>(nwg)),
                       dim3(64 * (kGdnScanWaves + 3)), 0,
                       stream, cu, n_tok, max_len, nchunk_cap, nseq, Hq, Hv, scale, q, k, v, g, ws, s0, o, s_out);
    return hipGetLastError();
}

size_t gdn_workspace_bytes(int nseq, int64_t max_len, int Hq, int Hv) {
    const int64_t nchunk_cap = (max_len + kGdnChunk - 1) / kGdnChunk;
    return static_cast<size_t>(nseq) * (Hv + Hq) * nchunk_cap * 2 * kGdnTile * sizeof(bf16_t);
}

}  // namespace qsa
