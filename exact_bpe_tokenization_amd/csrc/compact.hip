// compact.hip -- output compaction: per-piece ID runs -> one contiguous ID array per batch.
//
// TokTier (arXiv 2607.29678), GPU full-tokenization paragraph: the complete path ends with output
// compaction, and piece counts and output length stay in device memory (no host round trip between
// kernels).  Here: a single-pass exclusive scan of the per-piece token counts (decoupled look-back,
// dynamic tile ids), a gather of each piece's IDs into place, and the per-document token offsets
// (a document starts at the first piece whose start byte is >= its byte offset).
#include "internal.h"

namespace tt {

// tokoff[i] = sum of ntok[0..i) for i in [0, P]; tokoff[P] is the batch's token count
__global__ __launch_bounds__(SCAN_THREADS) void k_tokscan(uint8_t *ws, Layout L)
{
    __shared__ uint32_t s_tile, s_base;
    __shared__ uint32_t swsum[SCAN_THREADS / 64];
    Ctrl *ctrl = (Ctrl *)(ws + L.ctrl);
    const uint32_t *ntok = (const uint32_t *)(ws + L.ntok);
    uint32_t *tokoff = (uint32_t *)(ws + L.tokoff);
    uint64_t *flags = (uint64_t *)(ws + L.sflag);
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wid = tid >> 6;
    if (tid == 0) s_tile = atomicAdd(&ctrl->tile_ctr_scan, 1u);
    __syncthreads();
    const uint32_t tile = s_tile;
    const uint32_t np = ctrl->n_pieces;
    const uint64_t first = (uint64_t)tile * SCAN_TILE;
    if (first > np) return;                       // nothing at or below P in this tile
    const uint64_t i0 = first + (uint64_t)tid * SCAN_PER_THREAD;
    uint32_t x[SCAN_PER_THREAD], sum = 0;
    if (i0 + SCAN_PER_THREAD <= np) {
#pragma unroll
        for (int k = 0; k < SCAN_PER_THREAD; k += 4) {
            const uint4 w = *(const uint4 *)(ntok + i0 + k);
            x[k] = w.x; x[k + 1] = w.y; x[k + 2] = w.z; x[k + 3] = w.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < SCAN_PER_THREAD; ++k) x[k] = i0 + k < np ? ntok[i0 + k] : 0u;
    }
#pragma unroll
    for (int k = 0; k < SCAN_PER_THREAD; ++k) sum += x[k];
    uint32_t inc = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t y = __shfl_up(inc, d, 64);
        if (lane >= (uint32_t)d) inc += y;
    }
    if (lane == 63) swsum[wid] = inc;
    __syncthreads();
    uint32_t before = inc - sum, total = 0;
    for (uint32_t w = 0; w < SCAN_THREADS / 64; ++w) {
        if (w < wid) before += swsum[w];
        total += swsum[w];
    }
    if (wid == 0) {
        if (lane == 0 && tile > 0) st_flag(flags + tile, (1ull << 62) | total);
        const uint64_t basev = tile == 0 ? 0 : lookback_sum(flags, tile);
        if (lane == 0) {
            st_flag(flags + tile, (2ull << 62) | (basev + total));
            s_base = (uint32_t)basev;
        }
    }
    __syncthreads();
    uint32_t run = s_base + before;
#pragma unroll
    for (int k = 0; k < SCAN_PER_THREAD; ++k) {
        uint64_t i = i0 + k;
        if (i <= np) tokoff[i] = run;
        if (i == np) ctrl->n_tokens = run;
        run += x[k];
    }
}

__global__ __launch_bounds__(256) void k_gather(uint8_t *ws, Layout L, uint32_t *__restrict__ out_ids)
{
    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    const uint32_t *ntok = (const uint32_t *)(ws + L.ntok);
    const uint32_t *tokoff = (const uint32_t *)(ws + L.tokoff);
    const uint32_t *scratch = (const uint32_t *)(ws + L.scratch);
    const uint32_t np = ctrl->n_pieces;
    for (uint32_t p = blockIdx.x * blockDim.x + threadIdx.x; p < np; p += gridDim.x * blockDim.x) {
        const uint32_t b0 = pstart[p];
        if (pstart[p + 1] - b0 > LANE_MAX) continue;       // binned pieces: k_gather_long
        const uint32_t *src = scratch + b0;
        uint32_t *dst = out_ids + tokoff[p];
        const uint32_t c = ntok[p];
        for (uint32_t j = 0; j < c; ++j) dst[j] = src[j];
    }
}

// one workgroup per binned (longer than a lane's limit) piece
__global__ __launch_bounds__(256) void k_gather_long(uint8_t *ws, Layout L, uint32_t *__restrict__ out_ids)
{
    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    const uint32_t *ntok = (const uint32_t *)(ws + L.ntok);
    const uint32_t *tokoff = (const uint32_t *)(ws + L.tokoff);
    const uint32_t *scratch = (const uint32_t *)(ws + L.scratch);
    const uint32_t c0 = ctrl->bin_count[0], c1 = ctrl->bin_count[1], c2 = ctrl->bin_count[2];
    const uint32_t *l0 = (const uint32_t *)(ws + L.bin_wave), *l1 = (const uint32_t *)(ws + L.bin_block),
                   *l2 = (const uint32_t *)(ws + L.bin_giant);
    for (uint32_t q = blockIdx.x; q < c0 + c1 + c2; q += gridDim.x) {
        const uint32_t p = q < c0 ? l0[q] : (q < c0 + c1 ? l1[q - c0] : l2[q - c0 - c1]);
        const uint32_t *src = scratch + pstart[p];
        uint32_t *dst = out_ids + tokoff[p];
        const uint32_t c = ntok[p];
        for (uint32_t j = threadIdx.x; j < c; j += blockDim.x) dst[j] = src[j];
    }
}

__global__ __launch_bounds__(256) void k_docoff(uint8_t *ws, Layout L, const uint64_t *__restrict__ offsets,
                                               uint32_t n_docs, uint64_t *__restrict__ out_offsets)
{
    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    const uint32_t *tokoff = (const uint32_t *)(ws + L.tokoff);
    const uint32_t np = ctrl->n_pieces;
    for (uint64_t d = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; d <= n_docs;
         d += (uint64_t)gridDim.x * blockDim.x) {
        const uint64_t off = offsets[d];
        uint32_t a = 0, b = np;
        while (a < b) {
            uint32_t m = (a + b) >> 1;
            if ((uint64_t)pstart[m] < off) a = m + 1; else b = m;
        }
        out_offsets[d] = tokoff[a];
    }
}

__global__ __launch_bounds__(256) void k_export_starts(uint8_t *ws, Layout L, uint64_t n, uint32_t *out)
{
    const Ctrl *ctrl = (const Ctrl *)(ws + L.ctrl);
    const uint32_t *pstart = (const uint32_t *)(ws + L.pstart);
    const uint32_t np = ctrl->n_pieces;
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i <= np; i += gridDim.x * blockDim.x)
        out[i] = i == np ? (uint32_t)n : pstart[i];
}

hipError_t launch_compact(const Batch &b, uint32_t *out_ids, uint64_t *out_offsets, hipStream_t s,
                          const Events *ev)
{
    const Layout &L = b.L;
    {
        LaunchScope k(ev, 8, s);
        hipLaunchKernelGGL(k_tokscan, dim3(L.n_scan_tiles), dim3(SCAN_THREADS), 0, s, b.ws, L);
    }
    if (b.n) {
        LaunchScope k(ev, 9, s);
        uint32_t g = (uint32_t)((b.n + 255) / 256);
        hipLaunchKernelGGL(k_gather, dim3(g > 4096 ? 4096 : g), dim3(256), 0, s, b.ws, L, out_ids);
        uint32_t gl = L.cap_wave < 2048 ? L.cap_wave : 2048;
        hipLaunchKernelGGL(k_gather_long, dim3(gl), dim3(256), 0, s, b.ws, L, out_ids);
    }
    {
        LaunchScope k(ev, 10, s);
        uint32_t gd = (uint32_t)((b.n_docs + 1 + 255) / 256);
        hipLaunchKernelGGL(k_docoff, dim3(gd > 1024 ? 1024 : gd), dim3(256), 0, s, b.ws, L, b.offsets, b.n_docs,
                           out_offsets);
    }
    return hipGetLastError();
}

hipError_t launch_export_starts(const Batch &b, uint32_t *out_starts, hipStream_t s)
{
    uint32_t g = (uint32_t)((b.n + 1 + 255) / 256);
    hipLaunchKernelGGL(k_export_starts, dim3(g > 4096 ? 4096 : g), dim3(256), 0, s, b.ws, b.L, b.n, out_starts);
    return hipGetLastError();
}

}  // namespace tt
