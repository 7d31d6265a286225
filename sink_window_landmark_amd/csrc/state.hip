// State kernels: the empty state, the end of a call (accumulator scan, ring
// commit, meta) and the rewind of one push.  cortiq-engine 0.8.51
// src/gpu_wgpu/o1_batch.rs, o1b_far_commit, o1b_ring_commit and o1b_meta,
// applied to all rows of a call at once.
#include "swl_internal.h"
#include "stages.h"

namespace swl {

struct Windows {
    uint32_t w[64];
};

// meta = {0, 0, 0, window}, M = -inf, Z = 0, Theta = 0.
__global__ void k_init(KParams p, Windows win)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nth = (int64_t)p.nh * p.m * p.dv;
    const int64_t nmz = (int64_t)p.nh * 2 * p.m;
    if (idx < nth) p.theta[idx] = 0.f;
    if (idx < nmz) p.mz[idx] = ((idx / p.m) % 2 == 0) ? -INFINITY : 0.f;
    if (idx < p.G * 4) {
        const int g = (int)(idx / 4), f = (int)(idx % 4);
        p.meta[idx] = f == 3 ? win.w[g] : 0u;
    }
}

// The end of a call in one launch: (with `nth` > 0) the accumulator scan
// with its commit, the ring commit, and the meta update (stages.h).  Blocks
// [0, nth) scan, the next ring_blocks(p) commit rows, and the last one
// writes the meta.  None depends on another: every reader of the old ring
// rows and meta ran in earlier launches, and these read the call-start meta
// from its copy (p.meta).
__global__ __launch_bounds__(256) void k_commit(KParams p, int nth)
{
    const int64_t b = blockIdx.x;
    const int64_t nring = ring_blocks(p);
    if (b < nth) theta_scan_body(p, true, b);
    else if (b < nth + nring) ring_body(p, b - nth);
    else meta_body(p);
}

hipError_t launch_init(const KParams& p, const uint32_t* windows, hipStream_t st)
{
    Windows w{};
    for (int g = 0; g < p.G; ++g) w.w[g] = windows ? windows[g] : 0u;
    int64_t n = (int64_t)p.nh * p.m * p.dv;
    int64_t n2 = (int64_t)p.nh * 2 * p.m;
    if (n2 > n) n = n2;
    if (p.G * 4 > n) n = p.G * 4;
    hipLaunchKernelGGL(k_init, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, w);
    return hipGetLastError();
}

hipError_t launch_commit(const KParams& p, bool theta, hipStream_t st)
{
    const int64_t nth = theta ? theta_blocks(p) : 0;
    // without the scan (256 threads per block) the ring rows take one wave
    // each, so that every block of a long pass is resident at once
    hipLaunchKernelGGL(k_commit, dim3((unsigned)(nth + ring_blocks(p) + 1)), dim3(theta ? 256 : 64), 0, st, p,
                       (int)nth);
    return hipGetLastError();
}

// The bookkeeping of one push undone, per group (dory.rs dory_o1_back).  A
// push that evicted left the window full with at least one far key: its
// inverse moves the head back one slot and gives back one far count.  Any
// other push (the one that filled the window included: it evicted nothing,
// so the far count is still 0) only lengthened the window, which loses its
// newest row.  The ring's rows and M, Z, Theta stay as they are.  An empty
// window is left alone.
__global__ void k_rewind(KParams p)
{
    const int g = blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= p.G) return;
    const GMeta c = load_gmeta(p.meta, g, p.W);
    if (c.len0 == c.wg && c.nfar0 > 0) {
        p.meta[4 * g + 1] = (uint32_t)((c.head0 + c.wg - 1) % c.wg);
        p.meta[4 * g + 2] = (uint32_t)(c.nfar0 - 1);
    } else if (c.len0 > 0) {
        p.meta[4 * g + 0] = (uint32_t)(c.len0 - 1);
    }
}

hipError_t launch_rewind(const KParams& p, hipStream_t st)
{
    hipLaunchKernelGGL(k_rewind, dim3((p.G + 63) / 64), dim3(64), 0, st, p);
    return hipGetLastError();
}

}  // namespace swl
