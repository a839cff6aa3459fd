// Gather-rate probe of the benchmark: the memory traffic of the sparse
// attention's walk with its arithmetic taken out.  It is not part of the QSA
// boundary (include/qsa.h); bench.py uses it to measure, on the same GPU and
// in the same run, the rate at which 2 KiB micro-blocks can be gathered:
//   * from a region that fits in the L2 (the ceiling of any gather),
//   * uniformly at random from a cache as large as the workload's (no reuse),
//   * along the attention's own selection lists (its access stream alone).
//
// One wave per (row, KV group) list, four rows of one group per work-group and
// every work-group of group 0 before those of group 1, as the attention walk.
// A step gathers the K~ and V blocks of a few list entries with 16-byte loads
// per lane; the loaded words are folded into one checksum per wave so that no
// load is dead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int64_t kBlockBytes = 2048;

// kStep list entries per step: each entry's K~ and V blocks are loaded as
// 1 KiB halves, one 16-byte load per lane (lane l: bytes 16 l of the half),
// all of a step's loads issued before any is consumed.  kPadKiB KiB of LDS per
// work-group, touched once per lane (a volatile round trip of the checksum
// keeps it allocated), caps the work-groups a CU holds (160 KiB per CU).
template <int kStep, int kPadKiB>
__global__ __launch_bounds__(256) void gather_probe_kernel(const char *__restrict__ k_base,
                                                           const char *__restrict__ v_base, int64_t grp_stride,
                                                           int64_t n_blocks, const int32_t *__restrict__ idx,
                                                           int64_t rows, int64_t row0, int list_len,
                                                           uint32_t *__restrict__ sink)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t nt = (rows + 3) / 4;
    const int64_t x = blockIdx.x;
    const int grp = x >= nt ? 1 : 0;
    const int64_t r = (x - grp * nt) * 4 + wave;
    if (r >= rows) return;
    const int32_t *list = idx + (row0 + r) * list_len;
    const char *kb = k_base + grp * grp_stride + 16 * lane;
    const char *vb = v_base + grp * grp_stride + 16 * lane;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int c = 0; c + kStep <= list_len; c += kStep) {
        int64_t blk[kStep];
        for (int e = 0; e < kStep; ++e) {
            const int32_t id = list[c + e];
            blk[e] = (id >= 0 && id < n_blocks) ? id : 0;
        }
        u32x4 kf[kStep][2], vf[kStep][2];
        for (int e = 0; e < kStep; ++e)
            for (int hf = 0; hf < 2; ++hf) {
                kf[e][hf] = *reinterpret_cast<const u32x4 *>(kb + blk[e] * kBlockBytes + 1024 * hf);
                vf[e][hf] = *reinterpret_cast<const u32x4 *>(vb + blk[e] * kBlockBytes + 1024 * hf);
            }
        for (int e = 0; e < kStep; ++e)
            for (int hf = 0; hf < 2; ++hf) acc ^= kf[e][hf] ^ vf[e][hf];
    }
    uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
    for (int off = 32; off > 0; off >>= 1) v ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off));
    if constexpr (kPadKiB > 0) {
        __shared__ uint32_t pad[kPadKiB * 256];
        volatile uint32_t *pp = pad;
        pp[threadIdx.x] = v;
        v = pp[threadIdx.x];
    }
    if (lane == 0) sink[(grp * nt * 4 + r) & 0xFFFF] = v;
}

template <int kStep>
hipError_t launch_probe(hipStream_t st, dim3 grid, int pad_kib, const char *k_base, const char *v_base,
                        int64_t grp_stride, int64_t n_blocks, const int32_t *idx, int64_t n, int64_t r0, int list_len,
                        uint32_t *sink)
{
    switch (pad_kib) {
    case 0:
        hipLaunchKernelGGL((gather_probe_kernel<kStep, 0>), grid, dim3(256), 0, st, k_base, v_base, grp_stride,
                           n_blocks, idx, n, r0, list_len, sink);
        break;
    case 40:
        hipLaunchKernelGGL((gather_probe_kernel<kStep, 40>), grid, dim3(256), 0, st, k_base, v_base, grp_stride,
                           n_blocks, idx, n, r0, list_len, sink);
        break;
    case 64:
        hipLaunchKernelGGL((gather_probe_kernel<kStep, 64>), grid, dim3(256), 0, st, k_base, v_base, grp_stride,
                           n_blocks, idx, n, r0, list_len, sink);
        break;
    default:
        hipLaunchKernelGGL((gather_probe_kernel<kStep, 96>), grid, dim3(256), 0, st, k_base, v_base, grp_stride,
                           n_blocks, idx, n, r0, list_len, sink);
        break;
    }
    return hipGetLastError();
}

}  // namespace

extern "C" {

// Gather `rows` lists of `list_len` block ids (idx, int32 [rows][list_len],
// device) for both KV groups: group g reads the 2 KiB blocks at
// k_base + g*grp_stride + id*2048 and v_base + g*grp_stride + id*2048 for ids in
// [0, n_blocks) (other ids read block 0).  Launches of at most launch_rows rows
// on `stream` (a hipStream_t); sink is a device buffer of 65,536 uint32.
// step (2, 4 or 8) list entries are gathered per step; pad_kib (0, 40, 64 or
// 96) KiB of LDS per work-group caps the work-groups a CU holds, so the probe
// can run at the attention's occupancy.  Returns a hipError_t.
int qsa_probe_gather(void *stream, const void *k_base, const void *v_base, int64_t grp_stride, int64_t n_blocks,
                     const int32_t *idx, int64_t rows, int32_t list_len, int64_t launch_rows, int32_t step,
                     int32_t pad_kib, uint32_t *sink)
{
    if (!k_base || !v_base || !idx || !sink || rows < 0 || list_len < 0 || launch_rows <= 0 || n_blocks <= 0 ||
        (pad_kib != 0 && pad_kib != 40 && pad_kib != 64 && pad_kib != 96) || (step != 2 && step != 4 && step != 8))
        return static_cast<int>(hipErrorInvalidValue);
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (int64_t r0 = 0; r0 < rows; r0 += launch_rows) {
        const int64_t n = (r0 + launch_rows < rows) ? launch_rows : rows - r0;
        const dim3 grid(static_cast<unsigned>(2 * ((n + 3) / 4)));
        const char *kb = static_cast<const char *>(k_base), *vb = static_cast<const char *>(v_base);
        hipError_t e;
        if (step == 2)
            e = launch_probe<2>(st, grid, pad_kib, kb, vb, grp_stride, n_blocks, idx, n, r0, list_len, sink);
        else if (step == 4)
            e = launch_probe<4>(st, grid, pad_kib, kb, vb, grp_stride, n_blocks, idx, n, r0, list_len, sink);
        else
            e = launch_probe<8>(st, grid, pad_kib, kb, vb, grp_stride, n_blocks, idx, n, r0, list_len, sink);
        if (e != hipSuccess) return static_cast<int>(e);
    }
    return 0;
}

}  // extern "C"
