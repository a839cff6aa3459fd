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
// (chunk, V head) in parallel.  gdn_scan_kernel then walks the chunks of one
// (sequence, V head, 16*NW value columns) in order with its columns of S in
// registers (each column of S evolves on its own), so a head's state is
// advanced by 128/(16*NW) work-groups at once.
//
// Matrix cores: v_mfma_f32_16x16x32_bf16; A lane l = row l%16, k = 8(l/16)..+7;
// B lane l = column l%16, same k; C lane l = rows 4(l/16)..+3, column l%16.
// Accumulator tiles that feed a later product as its B operand (S, X, U) are
// rounded to bf16 and passed through a small per-wave LDS transpose.
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

// Workspace of one (sequence, V head, chunk): Tb then P, [64][64] bf16 each.
__device__ __forceinline__ int64_t gdn_ws_off(int s, int hv, int Hv, int nchunk_cap, int c) {
    return ((static_cast<int64_t>(s) * Hv + hv) * nchunk_cap + c) * (2 * kGdnTile);
}

// ---------------------------------------------------------------------------
// Per (chunk, QK head, sequence): K K^T and Q K^T of the chunk on the matrix
// cores (wave w owns rows 16w..16w+15, lower-triangular tiles only), then for
// each V head that reads this QK head: Lt into LDS and P to the workspace, and
// Tb by forward substitution, one column per lane (wave w solves head w of a
// group of up to four).
__global__ __launch_bounds__(256) void gdn_prep_kernel(const int32_t *__restrict__ cu, int64_t n_tok, int max_len,
                                                       int nchunk_cap, int Hq, int Hv, float scale,
                                                       const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
                                                       const float *__restrict__ g, const float *__restrict__ beta,
                                                       bf16_t *__restrict__ tp)
{
    __shared__ __align__(16) float smem[4 * kGdnTile];   // K, Q tiles; then Lt of up to four heads
    __shared__ float sG[4][kGdnChunk], sBeta[4][kGdnChunk];
    bf16_t *sK = reinterpret_cast<bf16_t *>(smem);
    bf16_t *sQ = sK + kGdnChunk * kGdnPad;

    const int c = blockIdx.x, hq = blockIdx.y, s = blockIdx.z;
    const GdnSpan sp = gdn_span(cu, s, n_tok, max_len);
    const int t0 = c * kGdnChunk;
    if (t0 >= sp.len) return;
    const int nt = min(kGdnChunk, sp.len - t0);
    const int rep = Hv / Hq;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;

    for (int p = tid; p < kGdnChunk * 16; p += 256) {
        const int t = p >> 4, d8 = p & 15;
        u32x4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
        if (t < nt) {
            const int64_t off = ((sp.base + t0 + t) * Hq + hq) * kGdnDim + d8 * 8;
            kv = *reinterpret_cast<const u32x4 *>(k + off);
            qv = *reinterpret_cast<const u32x4 *>(q + off);
        }
        *reinterpret_cast<u32x4 *>(sK + t * kGdnPad + d8 * 8) = kv;
        *reinterpret_cast<u32x4 *>(sQ + t * kGdnPad + d8 * 8) = qv;
    }
    __syncthreads();

    f32x4 kk[4], qk[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) kk[jt] = qk[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8 *>(sK + (16 * w + lr) * kGdnPad + 32 * s4 + 8 * lg);
        const bf16x8 aq = *reinterpret_cast<const bf16x8 *>(sQ + (16 * w + lr) * kGdnPad + 32 * s4 + 8 * lg);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            if (jt > w) continue;
            const bf16x8 bk = *reinterpret_cast<const bf16x8 *>(sK + (16 * jt + lr) * kGdnPad + 32 * s4 + 8 * lg);
            kk[jt] = mfma32(ak, bk, kk[jt]);
            qk[jt] = mfma32(aq, bk, qk[jt]);
        }
    }
    __syncthreads();   // K and Q tiles are dead: the space holds Lt from here on

    for (int r0 = 0; r0 < rep; r0 += 4) {
        const int nr = min(4, rep - r0);
        if (w < nr) {
            float gv = 0.f, bv = 0.f;
            if (lane < nt) {
                const int64_t gi = (sp.base + t0 + lane) * Hv + hq * rep + r0 + w;
                gv = g[gi];
                bv = beta[gi];
            }
            sG[w][lane] = wave_prefix_sum(gv);
            sBeta[w][lane] = bv;
        }
        __syncthreads();
        for (int r = 0; r < nr; ++r) {
            const int hv = hq * rep + r0 + r;
            bf16_t *P = tp + gdn_ws_off(s, hv, Hv, nchunk_cap, c) + kGdnTile;
            float *Lt = smem + r * kGdnTile;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int t = 16 * w + 4 * lg + j, jj = 16 * jt + lr;
                    float lv = 0.f, pv = 0.f;
                    if (jt <= w) {
                        const float Gj = sG[r][jj];
                        const float Gprev = t > 0 ? sG[r][t - 1] : 0.f;
                        if (jj < t) lv = sBeta[r][t] * expf(Gprev - Gj) * kk[jt][j];
                        if (jj <= t) pv = scale * expf(sG[r][t] - Gj) * qk[jt][j];
                        Lt[t * kGdnChunk + jj] = lv;   // tiles right of the diagonal are never read
                    }
                    P[t * kGdnChunk + jj] = f32_to_bf16(pv);
                }
            }
        }
        __syncthreads();
        if (w < nr) {
            // Column `lane` of T = (I + Lt)^{-1}: x_t = [t == lane] - sum_{j<t} Lt[t][j] x_j.
            // x_j is still zero for j >= t and so is Lt[t][j]: whole float4 reads are exact.
            const float *Lt = smem + w * kGdnTile;
            float x[kGdnChunk];
#pragma unroll
            for (int t = 0; t < kGdnChunk; ++t) x[t] = 0.f;
#pragma unroll
            for (int t = 0; t < kGdnChunk; ++t) {
                float acc = lane == t ? 1.f : 0.f;
#pragma unroll
                for (int j4 = 0; j4 < (t + 3) / 4; ++j4) {
                    const f32x4 l4 = *reinterpret_cast<const f32x4 *>(Lt + t * kGdnChunk + 4 * j4);
                    acc = fmaf(-l4[0], x[4 * j4 + 0], acc);
                    acc = fmaf(-l4[1], x[4 * j4 + 1], acc);
                    acc = fmaf(-l4[2], x[4 * j4 + 2], acc);
                    acc = fmaf(-l4[3], x[4 * j4 + 3], acc);
                }
                x[t] = acc;
            }
            const float bc = sBeta[w][lane];
            bf16_t *Tb = tp + gdn_ws_off(s, hq * rep + r0 + w, Hv, nchunk_cap, c);
#pragma unroll
            for (int t = 0; t < kGdnChunk; ++t) Tb[t * kGdnChunk + lane] = f32_to_bf16(x[t] * bc);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Chunk walk of one (sequence, V head, 16*NW value columns).  Wave w owns the
// 16 columns c0 = 16*(NW*slice + w) .. +15 of S (rows 16i + 4(l/16) + j of
// column c0 + l%16 in S[i][j]).  Per chunk, from LDS tiles shared by the waves:
//   R_K = K S, R_Q = Q S                 (32 products)
//   X = V - diag(gamma_{t-1}) R_K;  U = Tb X              (8)
//   O = diag(scale gamma_t) R_Q + P U                     (8)
//   S = gamma_C S + K^T diag(exp(G_C - G_t)) U            (16)
// The next chunk's tiles are loaded into registers while this one computes.
template <int NW>
struct GdnStage {
    static constexpr int NT = 64 * NW;
    static constexpr int kKd = 8 / NW;            // 16-byte K pieces per token of a thread
    static constexpr int kQp = 16 / NW;           // Q pieces of a thread
    static constexpr int kTp = 16 / NW;           // Tb + P pieces of a thread
    u32x4 ka[kKd], kb[kKd];                       // tokens 2*(tid%32) and +1, dims 8*(kKd*(tid/32) + m) ..
    u32x4 qv[kQp];
    u32x4 tpv[kTp];
    float gv;                                     // wave 0: g of token `lane`
    bf16_t vv[16];                                // this wave's V: tokens 16i + 4(l/16) + j, column c0 + l%16
};

template <int NW>
__global__ __launch_bounds__(64 * NW) void gdn_scan_kernel(const int32_t *__restrict__ cu, int64_t n_tok, int max_len,
                                                          int nchunk_cap, int Hq, int Hv, float scale,
                                                          const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
                                                          const bf16_t *__restrict__ v, const float *__restrict__ g,
                                                          const bf16_t *__restrict__ tp, const float *s0,
                                                          bf16_t *__restrict__ o, float *s_out)
{
    constexpr int NT = 64 * NW;
    constexpr int kSlices = kGdnDim / (16 * NW);
    __shared__ __align__(16) bf16_t sK[kGdnChunk * kGdnPad];
    __shared__ __align__(16) bf16_t sQ[kGdnChunk * kGdnPad];
    __shared__ __align__(16) bf16_t sKt[kGdnDim * kGdnPad64];
    __shared__ __align__(16) bf16_t sTb[kGdnChunk * kGdnPad64];
    __shared__ __align__(16) bf16_t sP[kGdnChunk * kGdnPad64];
    __shared__ __align__(16) bf16_t sTr[NW][16 * kGdnPad];
    __shared__ float sEp[kGdnChunk], sEc[kGdnChunk], sEt[kGdnChunk], sEC[1];

    // Work-groups are dealt to the 8 XCDs round-robin; renumber them so that the
    // column slices and V heads that share one QK head's tiles sit on one XCD.
    const int64_t nwg = gridDim.x;
    int64_t e = blockIdx.x;
    if (nwg % 8 == 0) e = (e % 8) * (nwg / 8) + e / 8;
    const int slice = static_cast<int>(e % kSlices);
    const int hv = static_cast<int>((e / kSlices) % Hv);
    const int s = static_cast<int>(e / (static_cast<int64_t>(kSlices) * Hv));
    const int hq = hv / (Hv / Hq);

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int col = 16 * (NW * slice + w) + lr;
    const GdnSpan sp = gdn_span(cu, s, n_tok, max_len);
    const int nck = (sp.len + kGdnChunk - 1) / kGdnChunk;
    const int64_t sbase = (static_cast<int64_t>(s) * Hv + hv) * kGdnDim * kGdnDim;

    f32x4 S[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            S[i][j] = s0 ? s0[sbase + static_cast<int64_t>(16 * i + 4 * lg + j) * kGdnDim + col] : 0.f;

    GdnStage<NW> st;
    auto load = [&](int c) {
        const int t0 = c * kGdnChunk;
        const int nt = min(kGdnChunk, sp.len - t0);
        const int tp2 = tid & 31, dg = tid >> 5;
#pragma unroll
        for (int m = 0; m < GdnStage<NW>::kKd; ++m) {
            const int d8 = dg * GdnStage<NW>::kKd + m;
            const int ta = 2 * tp2, tb = ta + 1;
            const bf16_t *src = k + ((sp.base + t0) * Hq + hq) * kGdnDim + d8 * 8;
            st.ka[m] = ta < nt ? *reinterpret_cast<const u32x4 *>(src + static_cast<int64_t>(ta) * Hq * kGdnDim)
                               : u32x4{0u, 0u, 0u, 0u};
            st.kb[m] = tb < nt ? *reinterpret_cast<const u32x4 *>(src + static_cast<int64_t>(tb) * Hq * kGdnDim)
                               : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int m = 0; m < GdnStage<NW>::kQp; ++m) {
            const int p = tid + NT * m, t = p >> 4, d8 = p & 15;
            st.qv[m] = t < nt ? *reinterpret_cast<const u32x4 *>(q + ((sp.base + t0 + t) * Hq + hq) * kGdnDim + d8 * 8)
                              : u32x4{0u, 0u, 0u, 0u};
        }
        const bf16_t *ws = tp + gdn_ws_off(s, hv, Hv, nchunk_cap, c);
#pragma unroll
        for (int m = 0; m < GdnStage<NW>::kTp; ++m)
            st.tpv[m] = *reinterpret_cast<const u32x4 *>(ws + 8 * (tid + NT * m));
        st.gv = (w == 0 && lane < nt) ? g[(sp.base + t0 + lane) * Hv + hv] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * i + 4 * lg + j;
                st.vv[4 * i + j] = t < nt ? v[((sp.base + t0 + t) * Hv + hv) * kGdnDim + col] : bf16_t(0);
            }
    };
    bf16_t vcur[16];
    auto store = [&]() {
        const int tp2 = tid & 31, dg = tid >> 5;
#pragma unroll
        for (int m = 0; m < GdnStage<NW>::kKd; ++m) {
            const int d8 = dg * GdnStage<NW>::kKd + m;
            *reinterpret_cast<u32x4 *>(sK + (2 * tp2) * kGdnPad + d8 * 8) = st.ka[m];
            *reinterpret_cast<u32x4 *>(sK + (2 * tp2 + 1) * kGdnPad + d8 * 8) = st.kb[m];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const uint32_t a = st.ka[m][e2], b = st.kb[m][e2];
                *reinterpret_cast<uint32_t *>(sKt + (d8 * 8 + 2 * e2) * kGdnPad64 + 2 * tp2) = (a & 0xFFFFu) | (b << 16);
                *reinterpret_cast<uint32_t *>(sKt + (d8 * 8 + 2 * e2 + 1) * kGdnPad64 + 2 * tp2) =
                    (a >> 16) | (b & 0xFFFF0000u);
            }
        }
#pragma unroll
        for (int m = 0; m < GdnStage<NW>::kQp; ++m) {
            const int p = tid + NT * m, t = p >> 4, d8 = p & 15;
            *reinterpret_cast<u32x4 *>(sQ + t * kGdnPad + d8 * 8) = st.qv[m];
        }
#pragma unroll
        for (int m = 0; m < GdnStage<NW>::kTp; ++m) {
            const int p = tid + NT * m;                  // 16-byte piece of [Tb; P]
            const int row = (p >> 3) & 63, c8 = p & 7;
            bf16_t *dst = (p < 512 ? sTb : sP) + row * kGdnPad64 + c8 * 8;
            *reinterpret_cast<u32x4 *>(dst) = st.tpv[m];
        }
        if (w == 0) {
            const float G = wave_prefix_sum(st.gv);
            const float Gprev = __shfl_up(G, 1);
            const float GC = __shfl(G, 63);
            sEp[lane] = lane == 0 ? 1.f : expf(Gprev);
            sEc[lane] = scale * expf(G);
            sEt[lane] = expf(GC - G);
            if (lane == 0) sEC[0] = expf(GC);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) vcur[i] = st.vv[i];
    };

    if (nck > 0) {
        load(0);
        store();
    }
    __syncthreads();
    bf16_t *tr = sTr[w];
    for (int c = 0; c < nck; ++c) {
        const int t0 = c * kGdnChunk;
        const int nt = min(kGdnChunk, sp.len - t0);
        if (c + 1 < nck) load(c + 1);

        // S -> bf16 B operand (k = rows of S).
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<u32x2 *>(tr + lr * kGdnPad + 16 * i + 4 * lg) =
                u32x2{pack_bf16x2(S[i][0], S[i][1]), pack_bf16x2(S[i][2], S[i][3])};
        wave_sync();
        bf16x8 bs[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) bs[s4] = *reinterpret_cast<const bf16x8 *>(tr + lr * kGdnPad + 32 * s4 + 8 * lg);
        f32x4 rk[4], rq[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rk[i] = rq[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                rk[i] = mfma32(*reinterpret_cast<const bf16x8 *>(sK + (16 * i + lr) * kGdnPad + 32 * s4 + 8 * lg),
                               bs[s4], rk[i]);
                rq[i] = mfma32(*reinterpret_cast<const bf16x8 *>(sQ + (16 * i + lr) * kGdnPad + 32 * s4 + 8 * lg),
                               bs[s4], rq[i]);
            }
        }
        // X = V - diag(gamma_{t-1}) K S, rows = tokens.
        wave_sync();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float xv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * i + 4 * lg + j;
                xv[j] = bf16_to_f32(vcur[4 * i + j]) - sEp[t] * rk[i][j];
            }
            *reinterpret_cast<u32x2 *>(tr + lr * kGdnPad + 16 * i + 4 * lg) =
                u32x2{pack_bf16x2(xv[0], xv[1]), pack_bf16x2(xv[2], xv[3])};
        }
        wave_sync();
        bf16x8 bx[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) bx[s2] = *reinterpret_cast<const bf16x8 *>(tr + lr * kGdnPad + 32 * s2 + 8 * lg);
        f32x4 U[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            U[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                U[i] = mfma32(*reinterpret_cast<const bf16x8 *>(sTb + (16 * i + lr) * kGdnPad64 + 32 * s2 + 8 * lg),
                              bx[s2], U[i]);
        }
        // U (for P U) in rows 0..63 and diag(exp(G_C - G_t)) U (for K^T) in rows 64..127.
        wave_sync();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tb = 16 * i + 4 * lg;
            *reinterpret_cast<u32x2 *>(tr + lr * kGdnPad + tb) =
                u32x2{pack_bf16x2(U[i][0], U[i][1]), pack_bf16x2(U[i][2], U[i][3])};
            *reinterpret_cast<u32x2 *>(tr + lr * kGdnPad + 64 + tb) =
                u32x2{pack_bf16x2(sEt[tb] * U[i][0], sEt[tb + 1] * U[i][1]),
                      pack_bf16x2(sEt[tb + 2] * U[i][2], sEt[tb + 3] * U[i][3])};
        }
        wave_sync();
        bf16x8 bu[2], bw[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            bu[s2] = *reinterpret_cast<const bf16x8 *>(tr + lr * kGdnPad + 32 * s2 + 8 * lg);
            bw[s2] = *reinterpret_cast<const bf16x8 *>(tr + lr * kGdnPad + 64 + 32 * s2 + 8 * lg);
        }
        // O = diag(scale gamma_t) Q S + P U
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 acc;
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = sEc[16 * i + 4 * lg + j] * rq[i][j];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                acc = mfma32(*reinterpret_cast<const bf16x8 *>(sP + (16 * i + lr) * kGdnPad64 + 32 * s2 + 8 * lg),
                             bu[s2], acc);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * i + 4 * lg + j;
                if (t < nt) o[((sp.base + t0 + t) * Hv + hv) * kGdnDim + col] = f32_to_bf16(acc[j]);
            }
        }
        // S = gamma_C S + K^T diag(exp(G_C - G_t)) U
        const float gC = sEC[0];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) S[i][j] *= gC;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                S[i] = mfma32(*reinterpret_cast<const bf16x8 *>(sKt + (16 * i + lr) * kGdnPad64 + 32 * s2 + 8 * lg),
                              bw[s2], S[i]);
        }
        __syncthreads();   // every wave is done with this chunk's tiles
        if (c + 1 < nck) store();
        __syncthreads();
    }
    if (s_out) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) s_out[sbase + static_cast<int64_t>(16 * i + 4 * lg + j) * kGdnDim + col] = S[i][j];
    }
}

constexpr int kGdnScanWaves = 2;

hipError_t launch_gdn_prefill(hipStream_t stream, int nseq, const int32_t *cu, int64_t n_tok, int max_len, int Hq,
                              int Hv, float scale, const bf16_t *q, const bf16_t *k, const bf16_t *v, const float *g,
                              const float *beta, const float *s0, bf16_t *o, float *s_out, bf16_t *tp)
{
    const int nchunk_cap = (max_len + kGdnChunk - 1) / kGdnChunk;
    if (nchunk_cap > 0) {
        hipLaunchKernelGGL(gdn_prep_kernel, dim3(static_cast<unsigned>(nchunk_cap), static_cast<unsigned>(Hq),
                                                 static_cast<unsigned>(nseq)),
                           dim3(256), 0, stream, cu, n_tok, max_len, nchunk_cap, Hq, Hv, scale, q, k, g, beta, tp);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    constexpr int kSlices = kGdnDim / (16 * kGdnScanWaves);
    const int64_t nwg = static_cast<int64_t>(nseq) * Hv * kSlices;
    hipLaunchKernelGGL(gdn_scan_kernel<kGdnScanWaves>, dim3(static_cast<unsigned>(nwg)), dim3(64 * kGdnScanWaves), 0,
                       stream, cu, n_tok, max_len, nchunk_cap, Hq, Hv, scale, q, k, v, g, tp, s0, o, s_out);
    return hipGetLastError();
}

size_t gdn_workspace_bytes(int nseq, int64_t max_len, int Hv) {
    const int64_t nchunk_cap = (max_len + kGdnChunk - 1) / kGdnChunk;
    return static_cast<size_t>(nseq) * Hv * nchunk_cap * 2 * kGdnTile * sizeof(bf16_t);
}

}  // namespace qsa
