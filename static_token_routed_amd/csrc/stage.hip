// Decode-path staging: one kernel copies the K / V rows of a step's distinct IDs
// from the tables in pinned host memory (read over PCIe through their device
// mapping) into compact device buffers.
//
// The pages keep the tables in host memory and move only the rows of the tokens
// just sampled to the GPU, overlapped with the layers that run before the lookup
// layer (sciencestack.ai page, Fig. 4 caption; papernotes.org page, section
// 关键设计 item 3).  Copying each contiguous run of rows with its own DMA
// request costs a few microseconds of set-up per run, and a step holds dozens of
// short runs; one kernel instead keeps many 16-byte PCIe reads in flight at once
// from every wavefront, and is bound by the link alone.
#include <algorithm>

#include "l3_internal.h"

namespace l3 {
namespace {

constexpr int kStageWaves = 4;  // wavefronts per workgroup
constexpr int kStageBatch = 4;  // chunks each lane has in flight per round

// Wavefront w copies destination rows w, w + W, ...: it finds the row's ID by a
// binary search over the compact offsets, then its lanes move the row's K part
// (rk chunks of sizeof(T) bytes) and V part (rv chunks) in rounds of kStageBatch
// loads followed by kStageBatch stores.  T is uint4 (16-byte chunks) when both row
// lengths are multiples of 16 bytes (every bf16 plan), else uint32_t (fp32 plans
// whose d_in or d_emb is not a multiple of 4).
// src[i] >= 0: the ID's first row in the host tables; src[i] < 0: its first row in
// the device-resident cache of hot rows is -1 - src[i] (cK, cV).
template <typename T>
__global__ __launch_bounds__(64 * kStageWaves) void k_stage_rows(
    const int64_t *__restrict__ coff, const int64_t *__restrict__ src, int64_t m, int64_t rows,
    const T *__restrict__ WK, const T *__restrict__ WV, const T *__restrict__ cK,
    const T *__restrict__ cV, T *__restrict__ dK, T *__restrict__ dV, int rk, int rv) {
    const int lane = threadIdx.x & 63;
    const int64_t nw = (int64_t)gridDim.x * kStageWaves;
    const int rt = rk + rv;
    for (int64_t r = (int64_t)blockIdx.x * kStageWaves + (threadIdx.x >> 6); r < rows; r += nw) {
        // last i with coff[i] <= r (coff[0] = 0, coff[m] = rows > r)
        int64_t lo = 0, hi = m;
        while (hi - lo > 1) {
            const int64_t mid = (lo + hi) >> 1;
            if (coff[mid] <= r) lo = mid; else hi = mid;
        }
        const int64_t s0 = src[lo];
        const bool cached = s0 < 0;
        const int64_t s = (cached ? -1 - s0 : s0) + (r - coff[lo]);
        const T *sk = (cached ? cK : WK) + s * rk, *sv = (cached ? cV : WV) + s * rv;
        T *tk = dK + r * rk, *tv = dV + r * rv;
        for (int c0 = 0; c0 < rt; c0 += 64 * kStageBatch) {
            T buf[kStageBatch];
#pragma unroll
            for (int j = 0; j < kStageBatch; ++j) {
                const int c = c0 + j * 64 + lane;
                if (c < rk) buf[j] = sk[c];
                else if (c < rt) buf[j] = sv[c - rk];
            }
#pragma unroll
            for (int j = 0; j < kStageBatch; ++j) {
                const int c = c0 + j * 64 + lane;
                if (c < rk) tk[c] = buf[j];
                else if (c < rt) tv[c - rk] = buf[j];
            }
        }
    }
}

}  // namespace

hipError_t launch_stage_rows(const int64_t *coff, const int64_t *src, int64_t m, int64_t rows,
                             const void *WK_dev, const void *WV_dev, const void *cK, const void *cV,
                             void *dK, void *dV, int64_t row_k_bytes, int64_t row_v_bytes,
                             hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    // enough wavefronts for a few hundred KB of reads in flight, and no more than
    // one per destination row
    const int64_t want = (rows + kStageWaves - 1) / kStageWaves;
    const int grid = (int)std::min<int64_t>(want, 1024);
    if (row_k_bytes % 16 == 0 && row_v_bytes % 16 == 0) {
        hipLaunchKernelGGL(k_stage_rows<uint4>, dim3(grid), dim3(64 * kStageWaves), 0, s, coff, src,
                           m, rows, (const uint4 *)WK_dev, (const uint4 *)WV_dev, (const uint4 *)cK,
                           (const uint4 *)cV, (uint4 *)dK, (uint4 *)dV, (int)(row_k_bytes / 16),
                           (int)(row_v_bytes / 16));
    } else {
        // row lengths are whole elements of 4 bytes (fp32) or 2 bytes (bf16, whose
        // dims are multiples of 64 and so never take this branch)
        hipLaunchKernelGGL(k_stage_rows<uint32_t>, dim3(grid), dim3(64 * kStageWaves), 0, s, coff,
                           src, m, rows, (const uint32_t *)WK_dev, (const uint32_t *)WV_dev,
                           (const uint32_t *)cK, (const uint32_t *)cV, (uint32_t *)dK,
                           (uint32_t *)dV, (int)(row_k_bytes / 4), (int)(row_v_bytes / 4));
    }
    return hipGetLastError();
}

}  // namespace l3
