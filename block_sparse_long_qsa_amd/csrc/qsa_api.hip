// Host side of the QSA C ABI: argument checks, workspace sizing and launch
// order.  Every check runs before the first launch, so a failing call leaves
// all buffers untouched.  The library never allocates device memory inside a
// call; the only device memory it owns is the handle's rotary tables.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "qsa.h"
#include "qsa_common.h"

namespace qsa {
void host_inv_freq(double theta, double yarn_factor, int64_t yarn_orig_ctx, double *out);
void host_rope_tables(const double *inv_freq, int64_t n_pos, float *cos_out, float *sin_out);

hipError_t launch_kv_pool(const Tables &, hipStream_t, int32_t, int64_t, int64_t, int64_t, const bf16_t *,
                          const bf16_t *, const bf16_t *, bf16_t *, bf16_t *, bf16_t *, const bf16_t *, bool, bool);
hipError_t launch_kpend_store(hipStream_t, int32_t, int64_t, int64_t, const bf16_t *, bf16_t *);
hipError_t launch_qidx_rotate(const Tables &, hipStream_t, int32_t, int64_t, int64_t, const int32_t *,
                              const bf16_t *, bf16_t *);
hipError_t launch_indexer_scores(hipStream_t, int32_t, int64_t, int64_t, int64_t, int64_t, const bf16_t *, int64_t,
                                 const bf16_t *, float *, int64_t, bool);
hipError_t launch_select(hipStream_t, int32_t, int64_t, int64_t, const int32_t *, int64_t, const float *, int64_t,
                         int32_t *, int64_t, int);
hipError_t launch_indexer_topk(hipStream_t, int32_t, int64_t, int64_t, int, int64_t, int, int, const bf16_t *, int64_t,
                               const bf16_t *, uint2 *, int32_t *, int64_t, int32_t *);
hipError_t launch_zero_words(hipStream_t, int32_t *, int64_t);
hipError_t launch_select_fixup(hipStream_t, int32_t, int64_t, int64_t, int, int, const int32_t *, int32_t *, int64_t,
                               const bf16_t *, int64_t, const bf16_t *, int64_t);
hipError_t launch_attend_prefill(const Tables &, hipStream_t, int32_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                                 int, float, const bf16_t *, const bf16_t *, const bf16_t *, const int32_t *,
                                 bf16_t *);
hipError_t launch_dense_attend(const Tables &, hipStream_t, int32_t, int64_t, int64_t, int64_t, int64_t, int64_t, float,
                               const bf16_t *, const bf16_t *, const bf16_t *, bf16_t *);
hipError_t launch_attend_decode(const Tables &, hipStream_t, int32_t, const int32_t *, const int32_t *, int64_t, int64_t,
                                int, int, float,
                                const bf16_t *, const bf16_t *, const bf16_t *, const int32_t *, float *, float *,
                                bf16_t *);
hipError_t launch_decode_append(const Tables &, hipStream_t, int32_t, const int32_t *, int64_t, int64_t, const bf16_t *,
                                const bf16_t *, const bf16_t *, bf16_t *, bf16_t *, bf16_t *, bf16_t *);
int64_t decode_scan_wgs(int64_t, int);
hipError_t launch_decode_scan(const Tables &, hipStream_t, int32_t, const int32_t *, int64_t, int, int64_t, int64_t, int,
                              int, const bf16_t *, bf16_t *, float *, uint32_t *, const bf16_t *, const bf16_t *,
                              const bf16_t *, bf16_t *, bf16_t *, bf16_t *, int64_t, uint2 *, uint32_t *);
hipError_t launch_select_list(hipStream_t, int32_t, const int32_t *, int64_t, int, const uint32_t *, int, int,
                              const uint2 *, const uint32_t *, int32_t *, int);
hipError_t launch_select_two_stage(hipStream_t, int32_t, const int32_t *, int64_t, int, int64_t, const float *,
                                   const uint32_t *, int, int, int32_t *, int32_t *, uint32_t *, int32_t *, uint32_t *,
                                   int32_t *, int);
hipError_t launch_attend_stats(const Tables &, hipStream_t, int32_t, int64_t, int64_t, int, float, const bf16_t *,
                               const bf16_t *, const bf16_t *, const int32_t *, bf16_t *, float *);
hipError_t launch_train_kl(const Tables &, hipStream_t, bool, int32_t, int64_t, int64_t, int, float, const bf16_t *,
                           const bf16_t *, const bf16_t *, const bf16_t *, const int32_t *, float *, float *,
                           const float *, float *, float *);
hipError_t launch_dk_idx(const Tables &, hipStream_t, int32_t, int64_t, int64_t, const float *, float *);
hipError_t launch_attend_backward(const Tables &, hipStream_t, int32_t, int64_t, int64_t, int, float, const bf16_t *,
                                  const bf16_t *, const bf16_t *, const int32_t *, const bf16_t *, const bf16_t *,
                                  const float *, float *, float *, float *);
hipError_t launch_token_keys(const Tables &, hipStream_t, int32_t, int64_t, int64_t, int64_t, const bf16_t *, bf16_t *);
hipError_t launch_gdn_prep(hipStream_t, int, const int32_t *, int64_t, int, int, int, float, const bf16_t *,
                           const bf16_t *, const float *, const float *, bf16_t *);
hipError_t launch_gdn_scan(hipStream_t, int, const int32_t *, int64_t, int, int, int, float, const bf16_t *,
                           const bf16_t *, const bf16_t *, const float *, const float *, bf16_t *, float *,
                           const bf16_t *);
size_t gdn_workspace_bytes(int, int64_t, int, int);

}  // namespace qsa

using namespace qsa;

struct qsa_handle {
    qsa_params p;
    int cap;            // candidate list length per query of the fused index + select stage
    int device;
    float *d_cos;
    float *d_sin;
    float sigma;        // softmax scale of the core logits
    char *scratch;      // device address of this device's no-allocation scratch array
};

namespace {

thread_local int g_last_hip = 0;

// Scratch of qsa_decode_noalloc: one array per GPU, held until the process
// ends.  In host code `scratch` is a stand-in for the symbol, not a device
// address: kernels and copies get the address hipGetSymbolAddress returns for
// the current device (kept in g_scratch per device, set by qsa_create).
static __device__ __align__(256) char scratch[QSA_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char *g_scratch[kMaxDevices] = {};

// The device address of the current device's scratch array (dev is current).
hipError_t scratch_address(int dev, char **out) {
    *out = nullptr;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = static_cast<char *>(p);
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

// Candidate lists of one fused index + select launch: at most this many bytes
// (the lists of 64 queries reserve 4 MiB at the default cap: 262,144 rows of
// one sequence in one launch, whose last work-groups are its shortest rows;
// in four 65,536-row launches each launch's tail left CUs idle, 15.24 against
// 14.86 ms at 262,144 tokens).
constexpr size_t kCandBytes = size_t(16) << 30;
constexpr int kDefaultCap = 8192;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

qsa_status hip_fail(hipError_t e) {
    g_last_hip = static_cast<int>(e);
    return QSA_ERR_HIP;
}

// Make the handle's device current for the duration of a call.
struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
        if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

Tables tables(const qsa_handle *h) { return Tables{h->d_cos, h->d_sin}; }
int64_t nblk_cap(const qsa_handle *h) { return h->p.max_ctx / kBlock; }

// Query rows of one fused index + select launch.
int64_t cand_rows(int32_t B, int64_t L, int cap) {
    const size_t per_row = static_cast<size_t>(B) * static_cast<size_t>(cap) * 8u;
    int64_t rows = static_cast<int64_t>(kCandBytes / per_row);
    rows = (rows / 64) * 64;
    if (rows < 64) rows = 64;
    return rows < L ? rows : L;
}

// Splits of the decode attention: about 512 waves (one wave per (sequence,
// KV group, split)); with its non-temporal gathers the walk measured faster
// in fewer, longer splits (512 to 768 waves) than at one wave per SIMD.
int decode_splits(int32_t B) {
    int s = (512 + 2 * B - 1) / (2 * B);
    return s < 1 ? 1 : (s > 32 ? 32 : s);
}

// Workspace of the fused index + select stage: rotated indexer queries, the
// candidate lists (score, block) of one launch of query rows, and the list of
// rows left to the exact fixup (a count, then b*rows + i per row).
struct IdxSelLayout { size_t qrot, cand, ovf, total; int64_t rows; };
IdxSelLayout index_select_layout(int32_t B, int64_t L, int cap) {
    IdxSelLayout f{};
    f.rows = cand_rows(B, L, cap);
    const size_t n = static_cast<size_t>(B) * f.rows;
    f.qrot = 0;
    f.cand = align_up(static_cast<size_t>(B) * L * kIdxHeads * kIdxDim * 2);
    f.ovf = f.cand + align_up(n * cap * 8);
    f.total = f.ovf + align_up((n + 1) * 4);
    return f;
}

// The decode selection handles rows of up to 1,024 chunks of 4,096 scores.
constexpr int64_t kDecodeChunkMax = 1024;

// Rows scanned by at most this many work-groups take their selection from the
// scan's candidate lists in one launch; longer rows use the two-stage path
// over the score rows.
constexpr int64_t kListMaxWG = 8;

struct DecLayout {
    size_t scores, bidx, part_o, part_ml, summ, s2cnt, s2gt, s2eqs, s2eqi, s2row, candn, total;
    int64_t ncol, nchunk, nwg;
    int nsplit, bpw;
    bool list;        // candidate lists (at scores, bpw (score, block) pairs per scan wave) instead of score rows
};

// Keys per wave of the decode scan: about one wave per SIMD over all rows
// (long streams per wave read faster than many short ones), a multiple of 64
// between 256 and kScanBlocksPerWaveMax.
int decode_scan_bpw(int32_t B, int64_t ncol) {
    const int64_t per = (static_cast<int64_t>(B) * ncol + 1023) / 1024;
    int64_t bpw = (per + 63) / 64 * 64;
    if (bpw < 256) bpw = 256;
    if (bpw > kScanBlocksPerWaveMax) bpw = kScanBlocksPerWaveMax;
    return static_cast<int>(bpw);
}
// rsh: log2 of the indexer's compression ratio (2: pooled micro-blocks; 0: tokens).
DecLayout decode_layout(const qsa_handle *h, int32_t B, int64_t ctx_bound, int rsh = 2) {
    DecLayout d{};
    d.ncol = ctx_bound >> rsh;
    if (d.ncol < 1) d.ncol = 1;
    d.nsplit = decode_splits(B);
    d.bpw = decode_scan_bpw(B, d.ncol);
    d.nwg = decode_scan_wgs(d.ncol, d.bpw);
    d.list = d.nwg <= kListMaxWG;
    d.scores = 0;
    d.bidx = d.scores + align_up(d.list ? static_cast<size_t>(B) * d.nwg * 4 * d.bpw * 8
                                        : static_cast<size_t>(B) * d.ncol * 4);
    d.part_o = d.bidx + align_up(static_cast<size_t>(B) * h->p.budget_blocks * 4);
    const size_t slots = static_cast<size_t>(B) * kKVHeads * d.nsplit * kGroup;
    d.part_ml = d.part_o + align_up(slots * kHeadDim * 4);
    // the scan work-groups' histogram summaries, one slot per (row, work-group)
    d.summ = d.part_ml + align_up(slots * 2 * 4);
    // two-stage selection: per 4,096-score chunk a count pair and the chunk's
    // lists (at most budget blocks above the boundary digit, 1,024 at it)
    d.nchunk = (d.ncol + 4095) / 4096;
    const size_t nck = d.list ? 0 : static_cast<size_t>(B) * d.nchunk;     // (the list path has no chunks)
    d.s2cnt = d.summ + align_up(static_cast<size_t>(B) * d.nwg * kSumSlot * 4);
    d.s2gt = d.s2cnt + align_up(nck * 2 * 4);
    d.s2eqs = d.s2gt + align_up(nck * kMaxBudget * 4);
    d.s2eqi = d.s2eqs + align_up(nck * 1024 * 4);
    d.s2row = d.s2eqi + align_up(nck * 1024 * 4);
    d.candn = d.s2row + align_up(static_cast<size_t>(B) * 3 * 4);
    d.total = d.candn + align_up(static_cast<size_t>(B) * d.nwg * 4 * 4);      // one count per scan wave
    return d;
}

// keys: pooled k̄ (rsh = 2, key_cap = max_ctx / 4) or token keys (rsh = 0, key_cap = max_ctx).
// The fused index + select launches for rows r_lo .. r_hi-1 of an L-row call
// whose indexer queries are already rotated into the workspace.
hipError_t index_select_rows(const qsa_handle *h, hipStream_t st, int32_t B, int64_t L, int64_t q_offset, int64_t r_lo,
                             int64_t r_hi, const uint16_t *kbar_cache, int32_t *bidx, char *w, const IdxSelLayout &f,
                             int rsh, int64_t key_cap) {
    const bf16_t *qrot = reinterpret_cast<const bf16_t *>(w + f.qrot);
    uint2 *cand = reinterpret_cast<uint2 *>(w + f.cand);
    int32_t *ovf = reinterpret_cast<int32_t *>(w + f.ovf);
    const int budget = h->p.budget_blocks;
    const int64_t qstride = L * kIdxHeads * kIdxDim;
    hipError_t e = hipSuccess;
    for (int64_t r0 = r_lo; r0 < r_hi && e == hipSuccess; r0 += f.rows) {
        const int64_t nr = (r0 + f.rows < r_hi) ? f.rows : r_hi - r0;
        const int64_t pos0 = q_offset + r0;
        const bf16_t *qr = qrot + r0 * kIdxHeads * kIdxDim;
        e = launch_zero_words(st, ovf, 1);
        if (e == hipSuccess)
            e = launch_indexer_topk(st, B, nr, pos0, rsh, key_cap, budget, h->cap, qr, qstride, kbar_cache, cand,
                                    bidx + r0 * budget, L * budget, ovf);
        if (e == hipSuccess)
            e = launch_select_fixup(st, B, nr, pos0, rsh, budget, ovf, bidx + r0 * budget, L * budget, qr, qstride,
                                    kbar_cache, key_cap);
    }
    return e;
}

hipError_t run_index_select(const qsa_handle *h, hipStream_t st, int32_t B, int64_t L, int64_t q_offset,
                            const uint16_t *q_idx, const uint16_t *kbar_cache, int32_t *bidx, char *w,
                            const IdxSelLayout &f, int rsh = 2, int64_t key_cap = -1) {
    if (key_cap < 0) key_cap = nblk_cap(h);
    bf16_t *qrot = reinterpret_cast<bf16_t *>(w + f.qrot);
    hipError_t e = launch_qidx_rotate(tables(h), st, B, L, q_offset, nullptr, q_idx, qrot);
    if (e == hipSuccess) e = index_select_rows(h, st, B, L, q_offset, 0, L, kbar_cache, bidx, w, f, rsh, key_cap);
    return e;
}

// The batch is a grid dimension (y or z) of every QSA kernel: at most 65,535.
constexpr int32_t kMaxBatch = 65535;

qsa_status check_chunk(const qsa_handle *h, int32_t B, int64_t L, int64_t q_offset, bool aligned_offset) {
    if (!h) return QSA_ERR_NULL;
    if (B < 1 || B > kMaxBatch || L < 0 || q_offset < 0) return QSA_ERR_SHAPE;
    if (aligned_offset && (q_offset % kBlock) != 0) return QSA_ERR_ALIGN;
    if (q_offset + L > h->p.max_ctx) return QSA_ERR_CAPACITY;
    return QSA_OK;
}

qsa_status check_ptrs(std::initializer_list<const void *> ptrs) {
    for (const void *p : ptrs)
        if (!p) return QSA_ERR_NULL;
    for (const void *p : ptrs)
        if (!aligned16(p)) return QSA_ERR_ALIGN;
    return QSA_OK;
}

// Host checks shared by the decode entry points (before anything is enqueued).
qsa_status check_decode(const qsa_handle *h, int32_t B, int64_t ctx_bound, std::initializer_list<const void *> ptrs,
                        const int32_t *block_idx) {
    if (!h) return QSA_ERR_NULL;
    if (B < 1 || B > kMaxBatch || ctx_bound < 0) return QSA_ERR_SHAPE;
    if (ctx_bound >= h->p.max_ctx) return QSA_ERR_CAPACITY;
    const qsa_status s = check_ptrs(ptrs);
    if (s != QSA_OK) return s;
    if (block_idx && !aligned16(block_idx)) return QSA_ERR_ALIGN;
    return QSA_OK;
}

// The selection half of a decode step with its scratch at w (layout d): the
// scan (whose first work-group per row appends the new token: K~/V when k is
// given, the indexer key pooled at r = 4 or rotated into the token keys at
// r = 1) -> the two-stage select from the scan's histogram summaries.
hipError_t run_decode_select(const qsa_handle *h, hipStream_t st, int32_t B, const int32_t *cache_len,
                             int64_t ctx_bound, int rsh, int64_t key_cap, const uint16_t *q_idx, uint16_t *keys,
                             const uint16_t *k, const uint16_t *v, const uint16_t *k_idx, uint16_t *k_cache,
                             uint16_t *v_cache, uint16_t *kpend, int32_t *bidx, char *w, const DecLayout &d) {
    float *scores = reinterpret_cast<float *>(w + d.scores);
    uint32_t *summ = reinterpret_cast<uint32_t *>(w + d.summ);
    uint2 *cand = d.list ? reinterpret_cast<uint2 *>(w + d.scores) : nullptr;
    uint32_t *candn = reinterpret_cast<uint32_t *>(w + d.candn);
    hipError_t e = launch_decode_scan(tables(h), st, B, cache_len, ctx_bound, rsh, key_cap, d.ncol,
                                      h->p.budget_blocks, d.bpw, q_idx, keys, scores, summ, k, v, k_idx, k_cache, v_cache,
                                      kpend, nblk_cap(h), cand, candn);
    if (d.list) {
        if (e == hipSuccess)
            e = launch_select_list(st, B, cache_len, ctx_bound, rsh, summ, static_cast<int>(d.nwg), d.bpw, cand, candn,
                                   bidx, h->p.budget_blocks);
        return e;
    }
    if (e == hipSuccess)
        e = launch_select_two_stage(st, B, cache_len, ctx_bound, rsh, d.ncol, scores, summ, static_cast<int>(d.nwg), d.bpw,
                                    reinterpret_cast<int32_t *>(w + d.s2cnt), reinterpret_cast<int32_t *>(w + d.s2gt),
                                    reinterpret_cast<uint32_t *>(w + d.s2eqs), reinterpret_cast<int32_t *>(w + d.s2eqi),
                                    reinterpret_cast<uint32_t *>(w + d.s2row), bidx, h->p.budget_blocks);
    return e;
}

// One decode step with its scratch at w (layout d): scan (+ append) ->
// two-stage select -> split-K attention -> merge.
hipError_t run_decode(const qsa_handle *h, hipStream_t st, int32_t B, const int32_t *cache_len, int64_t ctx_bound,
                      const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *q_idx,
                      const uint16_t *k_idx, uint16_t *k_cache, uint16_t *v_cache, uint16_t *kbar_cache,
                      uint16_t *kpend, uint16_t *out, int32_t *block_idx, char *w, const DecLayout &d) {
    int32_t *bidx = block_idx ? block_idx : reinterpret_cast<int32_t *>(w + d.bidx);
    float *part_o = reinterpret_cast<float *>(w + d.part_o);
    float *part_ml = reinterpret_cast<float *>(w + d.part_ml);
    const int64_t nbc = nblk_cap(h);
    hipError_t e = run_decode_select(h, st, B, cache_len, ctx_bound, 2, nbc, q_idx, kbar_cache, k, v, k_idx, k_cache,
                                     v_cache, kpend, bidx, w, d);
    if (e == hipSuccess)
        e = launch_attend_decode(tables(h), st, B, cache_len, nullptr, ctx_bound, nbc, h->p.budget_blocks, d.nsplit,
                                 h->sigma, q, k_cache, v_cache, bidx, part_o, part_ml, out);
    return e;
}

}  // namespace

extern "C" {

void qsa_default_params(qsa_params *p) {
    if (!p) return;
    memset(p, 0, sizeof(*p));
    p->n_q_heads = kQHeads;
    p->n_kv_heads = kKVHeads;
    p->head_dim = kHeadDim;
    p->rope_dim = kRopeDim;
    p->n_idx_heads = kIdxHeads;
    p->idx_dim = kIdxDim;
    p->idx_rope_dim = 64;
    p->block = kBlock;
    p->budget_blocks = kMaxBudget;
    p->max_ctx = 262144;
    p->rope_theta = 1e7;
    p->yarn_factor = 1.0;
    p->yarn_orig_ctx = 262144;
}

qsa_status qsa_create(const qsa_params *params, int device, qsa_handle **out) {
    if (!params || !out) return QSA_ERR_NULL;
    *out = nullptr;
    const qsa_params &p = *params;
    if (p.n_q_heads != kQHeads || p.n_kv_heads != kKVHeads || p.head_dim != kHeadDim || p.rope_dim != kRopeDim ||
        p.n_idx_heads != kIdxHeads || p.idx_dim != kIdxDim || p.idx_rope_dim != 64 || p.block != kBlock)
        return QSA_ERR_UNSUPPORTED;
    if (p.topk_cap != 0 && (p.topk_cap < 64 || p.topk_cap > kDefaultCap)) return QSA_ERR_SHAPE;
    if (p.budget_blocks < 1 || p.budget_blocks > kMaxBudget) return QSA_ERR_SHAPE;
    if (p.max_ctx < kBlock || p.max_ctx % kBlock != 0 || p.max_ctx > (int64_t(1) << 30)) return QSA_ERR_SHAPE;
    if (!(p.rope_theta > 1.0) || !isfinite(p.rope_theta)) return QSA_ERR_SHAPE;
    if (!(p.yarn_factor >= 1.0) || !isfinite(p.yarn_factor)) return QSA_ERR_SHAPE;
    if (p.yarn_factor > 1.0 && p.yarn_orig_ctx < 1) return QSA_ERR_SHAPE;

    double inv[kPairs];
    host_inv_freq(p.rope_theta, p.yarn_factor, p.yarn_orig_ctx, inv);
    const size_t n = static_cast<size_t>(p.max_ctx) * kPairs;
    std::vector<float> hc(n), hs(n);
    host_rope_tables(inv, p.max_ctx, hc.data(), hs.data());

    DeviceGuard guard(device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    qsa_handle *h = new (std::nothrow) qsa_handle();
    if (!h) return QSA_ERR_SHAPE;
    h->p = p;
    h->cap = p.topk_cap ? p.topk_cap : kDefaultCap;
    h->device = device;
    double sigma = 1.0 / sqrt(static_cast<double>(kHeadDim));
    if (p.yarn_factor > 1.0) {
        const double m = 0.1 * log(p.yarn_factor) + 1.0;
        sigma *= m * m;
    }
    h->sigma = static_cast<float>(sigma);
    hipError_t e = hipMalloc(reinterpret_cast<void **>(&h->d_cos), n * sizeof(float));
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&h->d_sin), n * sizeof(float));
    if (e == hipSuccess) e = scratch_address(device, &h->scratch);
    if (e == hipSuccess) e = hipMemcpy(h->d_cos, hc.data(), n * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(h->d_sin, hs.data(), n * sizeof(float), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        qsa_destroy(h);
        return hip_fail(e);
    }
    *out = h;
    return QSA_OK;
}

void qsa_destroy(qsa_handle *h) {
    if (!h) return;
    DeviceGuard guard(h->device);
    if (h->d_cos) (void)hipFree(h->d_cos);
    if (h->d_sin) (void)hipFree(h->d_sin);
    delete h;
}

qsa_status qsa_get_params(const qsa_handle *h, qsa_params *out) {
    if (!h || !out) return QSA_ERR_NULL;
    *out = h->p;
    return QSA_OK;
}

size_t qsa_workspace_size(const qsa_handle *h, int op, int32_t batch, int64_t len, int64_t q_offset) {
    if (!h || batch < 1 || len < 0 || q_offset < 0) return 0;
    switch (op) {
    case QSA_OP_APPEND:
    case QSA_OP_SELECT:
    case QSA_OP_ATTEND:
        return 0;
    case QSA_OP_INDEX:
        return align_up(static_cast<size_t>(batch) * len * kIdxHeads * kIdxDim * 2);
    case QSA_OP_INDEX_SELECT:
        return index_select_layout(batch, len, h->cap).total;
    case QSA_OP_FORWARD:
        return index_select_layout(batch, len, h->cap).total +
               align_up(static_cast<size_t>(batch) * len * h->p.budget_blocks * 4);
    case QSA_OP_DECODE:
    case QSA_OP_INDEX_DECODE:
        return decode_layout(h, batch, q_offset).total;
    case QSA_OP_TOKEN_INDEX_SELECT:
        return index_select_layout(batch, len, h->cap).total;
    case QSA_OP_TOKEN_INDEX_DECODE:
        return decode_layout(h, batch, q_offset, 0).total;
    case QSA_OP_TRAIN_FORWARD:
        return align_up(static_cast<size_t>(batch) * len * kIdxHeads * kIdxDim * 2);
    case QSA_OP_TRAIN_BACKWARD:
        return align_up(static_cast<size_t>(batch) * len * kIdxHeads * kIdxDim * 2) +
               align_up(static_cast<size_t>(batch) * nblk_cap(h) * kIdxDim * 4);
    default:
        return 0;
    }
}

qsa_status qsa_append(const qsa_handle *h, void *stream, int32_t B, int64_t L, int64_t q_offset,
                      const uint16_t *k, const uint16_t *v, const uint16_t *k_idx, uint16_t *k_cache,
                      uint16_t *v_cache, uint16_t *kbar_cache, uint16_t *kpend) {
    qsa_status s = check_chunk(h, B, L, q_offset, false);
    if (s != QSA_OK || L == 0) return s;
    if ((s = check_ptrs({k, v, k_idx, k_cache, v_cache, kbar_cache, kpend})) != QSA_OK) return s;
    DeviceGuard guard(h->device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = launch_kv_pool(tables(h), st, B, L, q_offset, nblk_cap(h), k, v, k_idx, k_cache, v_cache,
                                  kbar_cache, kpend, true, true);
    if (e == hipSuccess) e = launch_kpend_store(st, B, L, q_offset, k_idx, kpend);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

qsa_status qsa_index(const qsa_handle *h, void *stream, int32_t B, int64_t L, int64_t q_offset,
                     const uint16_t *q_idx, const uint16_t *kbar_cache, float *scores, void *ws, size_t ws_bytes) {
    qsa_status s = check_chunk(h, B, L, q_offset, true);
    if (s != QSA_OK || L == 0) return s;
    if ((s = check_ptrs({q_idx, kbar_cache, scores, ws})) != QSA_OK) return s;
    if (ws_bytes < qsa_workspace_size(h, QSA_OP_INDEX, B, L, q_offset)) return QSA_ERR_WORKSPACE;
    DeviceGuard guard(h->device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    hipStream_t st = static_cast<hipStream_t>(stream);
    bf16_t *qrot = static_cast<bf16_t *>(ws);
    const int64_t ncol = (q_offset + L + kBlock - 1) / kBlock;
    hipError_t e = launch_qidx_rotate(tables(h), st, B, L, q_offset, nullptr, q_idx, qrot);
    if (e == hipSuccess)
        e = launch_indexer_scores(st, B, L, q_offset, ncol, nblk_cap(h), qrot, L * kIdxHeads * kIdxDim, kbar_cache,
                                  scores, L * ncol, true);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

qsa_status qsa_select(const qsa_handle *h, void *stream, int32_t B, int64_t L, int64_t q_offset,
                      const float *scores, int32_t *block_idx) {
    qsa_status s = check_chunk(h, B, L, q_offset, true);
    if (s != QSA_OK || L == 0) return s;
    if ((s = check_ptrs({scores, block_idx})) != QSA_OK) return s;
    DeviceGuard guard(h->device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    const int64_t ncol = (q_offset + L + kBlock - 1) / kBlock;
    const int budget = h->p.budget_blocks;
    hipError_t e = launch_select(static_cast<hipStream_t>(stream), B, L, q_offset, nullptr, ncol, scores, L * ncol,
                                 block_idx, L * budget, budget);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

qsa_status qsa_attend(const qsa_handle *h, void *stream, int32_t B, int64_t L, int64_t q_offset, const uint16_t *q,
                      const uint16_t *k_cache, const uint16_t *v_cache, const int32_t *block_idx, uint16_t *out) {
    qsa_status s = check_chunk(h, B, L, q_offset, true);
    if (s != QSA_OK || L == 0) return s;
    if ((s = check_ptrs({q, k_cache, v_cache, block_idx, out})) != QSA_OK) return s;
    DeviceGuard guard(h->device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = launch_attend_prefill(tables(h), st, B, L, 0, L, q_offset, nblk_cap(h), h->p.budget_blocks, h->sigma, q,
                                  k_cache, v_cache, block_idx, out);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

qsa_status qsa_dense_attend(const qsa_handle *h, void *stream, int32_t B, int64_t L, int64_t q_offset,
                            const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache, uint16_t *out) {
    qsa_status s = check_chunk(h, B, L, q_offset, true);
    if (s != QSA_OK || L == 0) return s;
    if ((s = check_ptrs({q, k_cache, v_cache, out})) != QSA_OK) return s;
    DeviceGuard guard(h->device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    const hipError_t e = launch_dense_attend(tables(h), static_cast<hipStream_t>(stream), B, L, 0, L, q_offset,
                                             nblk_cap(h), h->sigma, q, k_cache, v_cache, out);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

qsa_status qsa_index_select(const qsa_handle *h, void *stream, int32_t B, int64_t L, int64_t q_offset,
                            const uint16_t *q_idx, const uint16_t *kbar_cache, int32_t *block_idx, void *ws,
                            size_t ws_bytes) {
    qsa_status s = check_chunk(h, B, L, q_offset, true);
    if (s != QSA_OK || L == 0) return s;
    if ((s = check_ptrs({q_idx, kbar_cache, block_idx, ws})) != QSA_OK) return s;
    const IdxSelLayout f = index_select_layout(B, L, h->cap);
    if (ws_bytes < f.total) return QSA_ERR_WORKSPACE;
    DeviceGuard guard(h->device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    hipError_t e = run_index_select(h, static_cast<hipStream_t>(stream), B, L, q_offset, q_idx, kbar_cache, block_idx,
                                    static_cast<char *>(ws), f);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

qsa_status qsa_forward(const qsa_handle *h, void *stream, int32_t B, int64_t L, int64_t q_offset, const uint16_t *q,
                       const uint16_t *k, const uint16_t *v, const uint16_t *q_idx, const uint16_t *k_idx,
                       uint16_t *k_cache, uint16_t *v_cache, uint16_t *kbar_cache, uint16_t *kpend, uint16_t *out,
                       int32_t *block_idx, void *ws, size_t ws_bytes) {
    qsa_status s = check_chunk(h, B, L, q_offset, true);
    if (s != QSA_OK || L == 0) return s;
    if ((s = check_ptrs({q, k, v, q_idx, k_idx, k_cache, v_cache, kbar_cache, kpend, out, ws})) != QSA_OK) return s;
    if (block_idx && !aligned16(block_idx)) return QSA_ERR_ALIGN;
    const IdxSelLayout f = index_select_layout(B, L, h->cap);
    const size_t bidx_off = f.total;
    const size_t total = bidx_off + align_up(static_cast<size_t>(B) * L * h->p.budget_blocks * 4);
    if (ws_bytes < total) return QSA_ERR_WORKSPACE;
    DeviceGuard guard(h->device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(ws);
    int32_t *bidx = block_idx ? block_idx : reinterpret_cast<int32_t *>(w + bidx_off);
    const int64_t nbc = nblk_cap(h);

    hipError_t e = launch_kv_pool(tables(h), st, B, L, q_offset, nbc, k, v, k_idx, k_cache, v_cache, kbar_cache,
                                  kpend, true, true);
    if (e == hipSuccess) e = launch_kpend_store(st, B, L, q_offset, k_idx, kpend);
    if (e == hipSuccess) e = run_index_select(h, st, B, L, q_offset, q_idx, kbar_cache, bidx, w, f);
    if (e == hipSuccess)
        e = launch_attend_prefill(tables(h), st, B, L, 0, L, q_offset, nbc, h->p.budget_blocks, h->sigma, q, k_cache,
                                  v_cache, bidx, out);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

qsa_status qsa_decode(const qsa_handle *h, void *stream, int32_t B, const int32_t *cache_len, int64_t ctx_bound,
                      const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *q_idx,
                      const uint16_t *k_idx, uint16_t *k_cache, uint16_t *v_cache, uint16_t *kbar_cache,
                      uint16_t *kpend, uint16_t *out, int32_t *block_idx, void *ws, size_t ws_bytes) {
    qsa_status s = check_decode(h, B, ctx_bound, {cache_len, q, k, v, q_idx, k_idx, k_cache, v_cache, kbar_cache,
                                                  kpend, out, ws}, block_idx);
    if (s != QSA_OK) return s;
    const DecLayout d = decode_layout(h, B, ctx_bound);
    if (d.nchunk > kDecodeChunkMax) return QSA_ERR_CAPACITY;
    if (ws_bytes < d.total) return QSA_ERR_WORKSPACE;
    DeviceGuard guard(h->device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    const hipError_t e = run_decode(h, static_cast<hipStream_t>(stream), B, cache_len, ctx_bound, q, k, v, q_idx,
                                    k_idx, k_cache, v_cache, kbar_cache, kpend, out, block_idx,
                                    static_cast<char *>(ws), d);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

qsa_status qsa_decode_noalloc(const qsa_handle *h, void *stream, int32_t B, const int32_t *cache_len,
                              int64_t ctx_bound, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const uint16_t *q_idx, const uint16_t *k_idx, uint16_t *k_cache, uint16_t *v_cache,
                              uint16_t *kbar_cache, uint16_t *kpend, uint16_t *out, int32_t *block_idx) {
    qsa_status s = check_decode(h, B, ctx_bound, {cache_len, q, k, v, q_idx, k_idx, k_cache, v_cache, kbar_cache,
                                                  kpend, out}, block_idx);
    if (s != QSA_OK) return s;
    const DecLayout d = decode_layout(h, B, ctx_bound);
    if (d.nchunk > kDecodeChunkMax) return QSA_ERR_CAPACITY;
    if (d.total > QSA_NOALLOC_SCRATCH_BYTES || !h->scratch) return QSA_ERR_WORKSPACE;
    DeviceGuard guard(h->device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    const hipError_t e = run_decode(h, static_cast<hipStream_t>(stream), B, cache_len, ctx_bound, q, k, v, q_idx,
                                    k_idx, k_cache, v_cache, kbar_cache, kpend, out, block_idx, h->scratch, d);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

qsa_status qsa_decode_reuse(const qsa_handle *h, void *stream, int32_t B, const int32_t *cache_len,
                            const int32_t *sel_pos, int64_t ctx_bound, const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const uint16_t *k_idx, uint16_t *k_cache, uint16_t *v_cache,
                            uint16_t *kbar_cache, uint16_t *kpend, const int32_t *block_idx, uint16_t *out, void *ws,
                            size_t ws_bytes) {
    if (!h) return QSA_ERR_NULL;
    if (B < 1 || B > kMaxBatch || ctx_bound < 0) return QSA_ERR_SHAPE;
    if (ctx_bound >= h->p.max_ctx) return QSA_ERR_CAPACITY;
    qsa_status s = check_ptrs({cache_len, sel_pos, q, k, v, k_idx, k_cache, v_cache, kbar_cache, kpend, block_idx, out,
                               ws});
    if (s != QSA_OK) return s;
    const DecLayout d = decode_layout(h, B, ctx_bound);
    if (d.nchunk > kDecodeChunkMax) return QSA_ERR_CAPACITY;
    if (ws_bytes < d.total) return QSA_ERR_WORKSPACE;
    DeviceGuard guard(h->device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(ws);
    float *part_o = reinterpret_cast<float *>(w + d.part_o);
    float *part_ml = reinterpret_cast<float *>(w + d.part_ml);
    const int64_t nbc = nblk_cap(h);
    hipError_t e = launch_decode_append(tables(h), st, B, cache_len, ctx_bound, nbc, k, v, k_idx, k_cache, v_cache,
                                        kbar_cache, kpend);
    if (e == hipSuccess)
        e = launch_attend_decode(tables(h), st, B, cache_len, sel_pos, ctx_bound, nbc, h->p.budget_blocks, d.nsplit,
                                 h->sigma, q, k_cache, v_cache, block_idx, part_o, part_ml, out);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

// Decode-step selection alone (r = 4): append the new token's indexer key
// (pending slot, pooling of a completed block), rotate the indexer query, scan
// the pooled keys and select -- the indexer half of qsa_decode.
qsa_status qsa_index_decode(const qsa_handle *h, void *stream, int32_t B, const int32_t *cache_len, int64_t ctx_bound,
                            const uint16_t *q_idx, const uint16_t *k_idx, uint16_t *kbar_cache, uint16_t *kpend,
                            int32_t *block_idx, void *ws, size_t ws_bytes) {
    if (!h) return QSA_ERR_NULL;
    if (B < 1 || B > kMaxBatch || ctx_bound < 0) return QSA_ERR_SHAPE;
    if (ctx_bound >= h->p.max_ctx) return QSA_ERR_CAPACITY;
    qsa_status s = check_ptrs({cache_len, q_idx, k_idx, kbar_cache, kpend, block_idx, ws});
    if (s != QSA_OK) return s;
    const DecLayout d = decode_layout(h, B, ctx_bound);
    if (d.nchunk > kDecodeChunkMax) return QSA_ERR_CAPACITY;
    if (ws_bytes < d.total) return QSA_ERR_WORKSPACE;
    DeviceGuard guard(h->device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(ws);
    const hipError_t e = run_decode_select(h, st, B, cache_len, ctx_bound, 2, nblk_cap(h), q_idx, kbar_cache, nullptr,
                                           nullptr, k_idx, nullptr, nullptr, kpend, block_idx, w, d);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

// Token-level indexer (r = 1): the O(n^2) indexer that QSA's pooled one
// replaces.  Same kernels with one rotated key per token and candidates t < p.
qsa_status qsa_token_index_select(const qsa_handle *h, void *stream, int32_t B, int64_t L, int64_t q_offset,
                                  const uint16_t *q_idx, const uint16_t *k_idx, uint16_t *ktok_cache,
                                  int32_t *token_idx, void *ws, size_t ws_bytes) {
    qsa_status s = check_chunk(h, B, L, q_offset, false);
    if (s != QSA_OK || L == 0) return s;
    if ((s = check_ptrs({q_idx, k_idx, ktok_cache, token_idx, ws})) != QSA_OK) return s;
    const IdxSelLayout f = index_select_layout(B, L, h->cap);
    if (ws_bytes < f.total) return QSA_ERR_WORKSPACE;
    DeviceGuard guard(h->device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = launch_token_keys(tables(h), st, B, L, q_offset, h->p.max_ctx, k_idx, ktok_cache);
    if (e == hipSuccess)
        e = run_index_select(h, st, B, L, q_offset, q_idx, ktok_cache, token_idx, static_cast<char *>(ws), f, 0,
                             h->p.max_ctx);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

qsa_status qsa_token_index_decode(const qsa_handle *h, void *stream, int32_t B, const int32_t *cache_len,
                                  int64_t ctx_bound, const uint16_t *q_idx, const uint16_t *k_idx,
                                  uint16_t *ktok_cache, int32_t *token_idx, void *ws, size_t ws_bytes) {
    if (!h) return QSA_ERR_NULL;
    if (B < 1 || B > kMaxBatch || ctx_bound < 0) return QSA_ERR_SHAPE;
    if (ctx_bound >= h->p.max_ctx) return QSA_ERR_CAPACITY;
    qsa_status s = check_ptrs({cache_len, q_idx, k_idx, ktok_cache, token_idx, ws});
    if (s != QSA_OK) return s;
    const DecLayout d = decode_layout(h, B, ctx_bound, 0);
    if (d.nchunk > kDecodeChunkMax) return QSA_ERR_CAPACITY;
    if (ws_bytes < d.total) return QSA_ERR_WORKSPACE;
    DeviceGuard guard(h->device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(ws);
    const hipError_t e = run_decode_select(h, st, B, cache_len, ctx_bound, 0, h->p.max_ctx, q_idx, ktok_cache,
                                           nullptr, nullptr, k_idx, nullptr, nullptr, nullptr, token_idx, w, d);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

// Training path: sparse attention + per-head log-sum-exp, then the indexer's
// KL loss against the max-pooled teacher (whole sequences: positions 0..L-1).
qsa_status qsa_train_forward(const qsa_handle *h, void *stream, int32_t B, int64_t L, const uint16_t *q,
                             const uint16_t *q_idx, const uint16_t *k_cache, const uint16_t *v_cache,
                             const uint16_t *kbar_cache, const int32_t *block_idx, uint16_t *out, float *stats,
                             float *kl, void *ws, size_t ws_bytes) {
    qsa_status s = check_chunk(h, B, L, 0, true);
    if (s != QSA_OK || L == 0) return s;
    if ((s = check_ptrs({q, q_idx, k_cache, v_cache, kbar_cache, block_idx, out, stats, kl, ws})) != QSA_OK) return s;
    if (ws_bytes < qsa_workspace_size(h, QSA_OP_TRAIN_FORWARD, B, L, 0)) return QSA_ERR_WORKSPACE;
    DeviceGuard guard(h->device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    hipStream_t st = static_cast<hipStream_t>(stream);
    bf16_t *qrot = static_cast<bf16_t *>(ws);
    const int64_t nbc = nblk_cap(h);
    const int budget = h->p.budget_blocks;
    hipError_t e = launch_qidx_rotate(tables(h), st, B, L, 0, nullptr, q_idx, qrot);
    if (e == hipSuccess)
        e = launch_attend_stats(tables(h), st, B, L, nbc, budget, h->sigma, q, k_cache, v_cache, block_idx, out, stats);
    if (e == hipSuccess)
        e = launch_train_kl(tables(h), st, false, B, L, nbc, budget, h->sigma, q, k_cache, kbar_cache, qrot, block_idx,
                            stats, kl, nullptr, nullptr, nullptr);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

qsa_status qsa_train_backward_indexer(const qsa_handle *h, void *stream, int32_t B, int64_t L, const uint16_t *q,
                                      const uint16_t *q_idx, const uint16_t *k_cache, const uint16_t *kbar_cache,
                                      const int32_t *block_idx, const float *stats, const float *dkl, float *dq_idx,
                                      float *dk_idx, void *ws, size_t ws_bytes) {
    qsa_status s = check_chunk(h, B, L, 0, true);
    if (s != QSA_OK || L == 0) return s;
    if ((s = check_ptrs({q, q_idx, k_cache, kbar_cache, block_idx, stats, dkl, dq_idx, dk_idx, ws})) != QSA_OK)
        return s;
    if (ws_bytes < qsa_workspace_size(h, QSA_OP_TRAIN_BACKWARD, B, L, 0)) return QSA_ERR_WORKSPACE;
    DeviceGuard guard(h->device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(ws);
    bf16_t *qrot = reinterpret_cast<bf16_t *>(w);
    float *dkbar = reinterpret_cast<float *>(w + align_up(static_cast<size_t>(B) * L * kIdxHeads * kIdxDim * 2));
    const int64_t nbc = nblk_cap(h);
    hipError_t e = launch_qidx_rotate(tables(h), st, B, L, 0, nullptr, q_idx, qrot);
    if (e == hipSuccess) e = launch_zero_words(st, reinterpret_cast<int32_t *>(dkbar), static_cast<int64_t>(B) * nbc * kIdxDim);
    if (e == hipSuccess)
        e = launch_train_kl(tables(h), st, true, B, L, nbc, h->p.budget_blocks, h->sigma, q, k_cache, kbar_cache, qrot,
                            block_idx, const_cast<float *>(stats), nullptr, dkl, dq_idx, dkbar);
    if (e == hipSuccess) e = launch_dk_idx(tables(h), st, B, L, nbc, dkbar, dk_idx);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

qsa_status qsa_train_backward_attention(const qsa_handle *h, void *stream, int32_t B, int64_t L, const uint16_t *q,
                                        const uint16_t *k_cache, const uint16_t *v_cache, const int32_t *block_idx,
                                        const uint16_t *out, const uint16_t *dout, const float *stats, float *dq,
                                        float *dk, float *dv) {
    qsa_status s = check_chunk(h, B, L, 0, true);
    if (s != QSA_OK || L == 0) return s;
    if ((s = check_ptrs({q, k_cache, v_cache, block_idx, out, dout, stats, dq, dk, dv})) != QSA_OK) return s;
    DeviceGuard guard(h->device);
    if (!guard.ok) return hip_fail(hipErrorInvalidDevice);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t n = static_cast<int64_t>(B) * L * kKVHeads * kHeadDim;
    hipError_t e = launch_zero_words(st, reinterpret_cast<int32_t *>(dk), n);
    if (e == hipSuccess) e = launch_zero_words(st, reinterpret_cast<int32_t *>(dv), n);
    if (e == hipSuccess)
        e = launch_attend_backward(tables(h), st, B, L, nblk_cap(h), h->p.budget_blocks, h->sigma, q, k_cache, v_cache,
                                   block_idx, out, dout, stats, dq, dk, dv);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

size_t qsa_gdn_workspace_size(int32_t nseq, int64_t max_len, int32_t hq_heads, int32_t hv_heads) {
    if (nseq < 1 || max_len < 0 || hq_heads < 1 || hv_heads < 1) return 0;
    return align_up(gdn_workspace_bytes(nseq, max_len, hq_heads, hv_heads));
}

namespace {
// Checks shared by the GDN entry points (everything before the first launch).
qsa_status gdn_check(int32_t nseq, const int32_t *cu, int64_t n_tokens, int64_t max_len, int32_t hq, int32_t hv,
                     std::initializer_list<const void *> needed, const void *q, const void *k, const void *ws,
                     size_t ws_bytes) {
    if (!cu) return QSA_ERR_NULL;
    for (const void *p : needed)
        if (!p) return QSA_ERR_NULL;
    if (nseq < 1 || nseq > 65535 || n_tokens < 0 || max_len < 0 || max_len > (int64_t(1) << 30) || hq < 1 ||
        hq > 65535 || hv < hq || hv % hq != 0)
        return QSA_ERR_SHAPE;
    // Launch grids: nseq * chunks * hv one-wave work-groups (prep), nseq * hv * 4 (scan).
    if (static_cast<int64_t>(nseq) * ((max_len + 63) / 64) * hv > int64_t(0xFFFFFFFF)) return QSA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k)) return QSA_ERR_ALIGN;
    const size_t need = qsa_gdn_workspace_size(nseq, max_len, hq, hv);
    if (need > 0) {
        if (!ws) return QSA_ERR_NULL;
        if (!aligned16(ws)) return QSA_ERR_ALIGN;
        if (ws_bytes < need) return QSA_ERR_WORKSPACE;
    }
    return QSA_OK;
}
}  // namespace

qsa_status qsa_gdn_chunk_prefill(void *stream, int32_t nseq, const int32_t *cu_seqlens, int64_t n_tokens,
                                 int64_t max_len, int32_t hq_heads, int32_t hv_heads, float scale, const uint16_t *q,
                                 const uint16_t *k, const uint16_t *v, const float *g, const float *beta,
                                 const float *initial_state, uint16_t *o, float *final_state, void *ws,
                                 size_t ws_bytes) {
    qsa_status s = gdn_check(nseq, cu_seqlens, n_tokens, max_len, hq_heads, hv_heads, {q, k, v, g, beta, o}, q, k, ws,
                             ws_bytes);
    if (s != QSA_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    bf16_t *tp = static_cast<bf16_t *>(ws);
    hipError_t e = launch_gdn_prep(st, nseq, cu_seqlens, n_tokens, static_cast<int>(max_len), hq_heads, hv_heads,
                                   scale, q, k, g, beta, tp);
    if (e == hipSuccess)
        e = launch_gdn_scan(st, nseq, cu_seqlens, n_tokens, static_cast<int>(max_len), hq_heads, hv_heads, scale, q,
                            k, v, g, initial_state, o, final_state, tp);
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

qsa_status qsa_gdn_prep(void *stream, int32_t nseq, const int32_t *cu_seqlens, int64_t n_tokens, int64_t max_len,
                        int32_t hq_heads, int32_t hv_heads, float scale, const uint16_t *q, const uint16_t *k,
                        const float *g, const float *beta, void *ws, size_t ws_bytes) {
    qsa_status s = gdn_check(nseq, cu_seqlens, n_tokens, max_len, hq_heads, hv_heads, {q, k, g, beta}, q, k, ws,
                             ws_bytes);
    if (s != QSA_OK) return s;
    hipError_t e = launch_gdn_prep(static_cast<hipStream_t>(stream), nseq, cu_seqlens, n_tokens,
                                   static_cast<int>(max_len), hq_heads, hv_heads, scale, q, k, g, beta,
                                   static_cast<bf16_t *>(ws));
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

qsa_status qsa_gdn_scan(void *stream, int32_t nseq, const int32_t *cu_seqlens, int64_t n_tokens, int64_t max_len,
                        int32_t hq_heads, int32_t hv_heads, float scale, const uint16_t *q, const uint16_t *k,
                        const uint16_t *v, const float *g, const float *initial_state, uint16_t *o,
                        float *final_state, const void *ws, size_t ws_bytes) {
    qsa_status s = gdn_check(nseq, cu_seqlens, n_tokens, max_len, hq_heads, hv_heads, {q, k, v, g, o}, q, k, ws,
                             ws_bytes);
    if (s != QSA_OK) return s;
    hipError_t e = launch_gdn_scan(static_cast<hipStream_t>(stream), nseq, cu_seqlens, n_tokens,
                                   static_cast<int>(max_len), hq_heads, hv_heads, scale, q, k, v, g, initial_state, o,
                                   final_state, static_cast<const bf16_t *>(ws));
    return e == hipSuccess ? QSA_OK : hip_fail(e);
}

const char *qsa_status_string(qsa_status s) {
    switch (s) {
    case QSA_OK: return "ok";
    case QSA_ERR_NULL: return "a required pointer is NULL";
    case QSA_ERR_SHAPE: return "a size or count is out of range";
    case QSA_ERR_UNSUPPORTED: return "head counts or dims other than the built ones";
    case QSA_ERR_ALIGN: return "pointer not 16-byte aligned or q_offset not a multiple of 4";
    case QSA_ERR_CAPACITY: return "positions beyond the cache capacity max_ctx";
    case QSA_ERR_WORKSPACE: return "workspace smaller than qsa_workspace_size()";
    case QSA_ERR_HIP: return "HIP runtime error (see qsa_last_hip_error)";
    default: return "unknown status";
    }
}

int qsa_last_hip_error(void) { return g_last_hip; }

}  // extern "C"
