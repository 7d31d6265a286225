// State kernels: the empty state, the ring commit and the ring bookkeeping.
// cortiq-engine 0.8.51 src/gpu_wgpu/o1_batch.rs, o1b_ring_commit and
// o1b_meta, applied to all rows of a call at once.
#include "swl_internal.h"

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

// Chunk row r of the call lands in slot (head0 + len0 + r) mod w_g, the
// slot its own eviction freed (o1b_ring_commit).  Only the last w_g rows of
// the call survive in the ring, so only they are written: that keeps the
// writes of a call whose rows outnumber the window free of collisions.
// One block per (row, group), rows counted back from the end of the call.
__global__ __launch_bounds__(256) void k_ring_commit(KParams p)
{
    const int g = blockIdx.y;
    const GMeta c = load_gmeta(p.meta, g, p.W);
    const int r = p.T - 1 - (int)blockIdx.x;
    if (r < 0 || r < p.T - c.wg) return;
    const int slot = (int)(((int64_t)c.head0 + c.len0 + r) % c.wg);
    const float* ks = p.k + ((int64_t)r * p.G + g) * p.d;
    const float* vs = p.v + ((int64_t)r * p.G + g) * p.dv;
    float* kd = p.ring_k + ((int64_t)g * p.W + slot) * p.d;
    float* vd = p.ring_v + ((int64_t)g * p.W + slot) * p.dv;
    const float* kt = p.rope ? p.rope + (int64_t)r * p.d : nullptr;   // the ring holds turned keys
    for (int t = threadIdx.x; t < p.d / 4; t += 256)
        reinterpret_cast<float4*>(kd)[t] = rope4(ks, kt, 4 * t, p.d);
    for (int t = threadIdx.x; t < p.dv / 4; t += 256)
        reinterpret_cast<float4*>(vd)[t] = reinterpret_cast<const float4*>(vs)[t];
}

// len, head and nfar after T pushes (o1b_meta with k = T).
__global__ void k_meta(KParams p)
{
    const int g = blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= p.G) return;
    const GMeta c = load_gmeta(p.meta, g, p.W);
    const int64_t tot = (int64_t)c.len0 + p.T;
    if (tot <= c.wg) {
        p.meta[4 * g + 0] = (uint32_t)tot;
    } else {
        const int64_t ev = tot - c.wg;
        p.meta[4 * g + 0] = (uint32_t)c.wg;
        p.meta[4 * g + 1] = (uint32_t)((c.head0 + ev) % c.wg);
        p.meta[4 * g + 2] = (uint32_t)(c.nfar0 + ev);
    }
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

hipError_t launch_ring_commit(const KParams& p, hipStream_t st)
{
    const int rows = p.T < p.W ? p.T : p.W;
    hipLaunchKernelGGL(k_ring_commit, dim3(rows, p.G), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_meta(const KParams& p, hipStream_t st)
{
    hipLaunchKernelGGL(k_meta, dim3((p.G + 63) / 64), dim3(64), 0, st, p);
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
