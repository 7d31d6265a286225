// Device bodies of the small stages of a call -- the far accumulator scan,
// the ring commit and the meta update -- so that one launch can run them
// beside another stage: each block takes its role from its index, and no
// block waits on another.  cortiq-engine 0.8.51 src/gpu_wgpu/o1_batch.rs,
// o1b_far_commit, o1b_ring_commit and o1b_meta.
#pragma once

#include "swl_internal.h"

namespace swl {

constexpr int SCAN_AHEAD = 32;   // sub-chunks of loads the accumulator scan keeps in flight

__device__ __forceinline__ void two_sum(float a, float b, float& s, float& e)
{
#pragma clang fp contract(off)
    s = a + b;
    const float bv = s - a;
    e = (a - (s - bv)) + (b - bv);
}

// Blocks of 256 threads the accumulator scan takes: a thread per element.
__host__ __device__ inline int64_t theta_blocks(const KParams& p)
{
    return ((int64_t)p.nh * p.m * p.dv + 255) / 256;
}

// theta_scan, block `bid` of theta_blocks(p): one thread per (gh, b, t),
// walking the sub-chunks in order: TH[s] <- Theta (the value before
// sub-chunk s, which the readout of s uses), Theta <- R_s Theta +
// fac_s dTheta_s (dtheta's increment is against the sub-chunk's own max;
// fac_s brings it to the post-sub-chunk max).
// With `commit` the final Theta, M and Z go to the state (o1b_far_commit:
// M <- M', Z <- the mass after the rows).
//
// Theta is carried as an unevaluated sum th + tc of two fp32 numbers
// (compensated summation): the rounding error of each product R_s th (an
// fma gives it exactly) and of each sum (Knuth's two-sum) goes into tc, so
// the running value keeps about twice fp32's precision over the hundreds of
// sub-chunks of a pass, and only its final rounding to one fp32 number
// (and each TH[s]) is left.  The element of an accumulator that sums tens
// of thousands of signed terms can cancel to a value far below the terms'
// scale; plain fp32 accumulation would leave there an error of order
// 2^-24 times the partial sums' magnitude per sub-chunk.
__device__ __forceinline__ void theta_scan_body(const KParams& p, bool commit, int64_t bid)
{
    // every product and sum below rounds on its own: a product fused into a
    // later sum would no longer be the value whose error the fma takes
#pragma clang fp contract(off)
    const int64_t nhm = (int64_t)p.nh * p.m;
    const int64_t idx = bid * 256 + threadIdx.x;
    if (idx >= nhm * p.dv) return;
    const int64_t ghb = idx / p.dv;
    const int64_t stride = nhm * p.dv;
    float th = p.theta[idx], tc = 0.f;
    for (int s0 = 0; s0 < p.S; s0 += SCAN_AHEAD) {
        float dth[SCAN_AHEAD], rs[SCAN_AHEAD], fs[SCAN_AHEAD];
#pragma unroll
        for (int k = 0; k < SCAN_AHEAD; ++k) {
            const int s = min(s0 + k, p.S - 1);
            dth[k] = p.TH[(int64_t)s * stride + idx];
            rs[k] = p.Rs[(int64_t)s * nhm + ghb];
            fs[k] = p.FAC[(int64_t)s * nhm + ghb];
        }
#pragma unroll
        for (int k = 0; k < SCAN_AHEAD; ++k) {
            const int s = s0 + k;
            if (s < p.S) {
                p.TH[(int64_t)s * stride + idx] = th;
                // (th + tc) R + fac d, with the errors of both products and
                // of the sum kept
                const float pr = rs[k] * th;
                const float pe = fmaf(rs[k], th, -pr);
                const float pd = fs[k] * dth[k];
                const float pde = fmaf(fs[k], dth[k], -pd);
                float sm, se;
                two_sum(pr, pd, sm, se);
                const float lo = fmaf(rs[k], tc, (pe + pde) + se);
                two_sum(sm, lo, th, tc);
            }
        }
    }
    if (commit) {
        p.theta[idx] = th;
        if (idx % p.dv == 0) {
            const int64_t gh = ghb / p.m, b = ghb % p.m;
            const int64_t last = (int64_t)(p.S - 1) * nhm + ghb;
            p.mz[gh * 2 * p.m + b] = p.Ms[last];
            p.mz[gh * 2 * p.m + p.m + b] = p.TZ[(int64_t)p.S * nhm + ghb];
        }
    }
}

// Blocks of the ring commit: one per (row, group) of the last min(T, W) rows.
__host__ __device__ inline int64_t ring_blocks(const KParams& p)
{
    return (int64_t)(p.T < p.W ? p.T : p.W) * p.G;
}

// Ring commit, block `bid` of ring_blocks(p) (256 threads): chunk row r of
// the call lands in slot (head0 + len0 + r) mod w_g, the slot its own
// eviction freed (o1b_ring_commit).  Only the last w_g rows of the call
// survive in the ring, so only they are written: that keeps the writes of a
// call whose rows outnumber the window free of collisions.  Rows are
// counted back from the end of the call.  p.meta is the call-start meta.
__device__ __forceinline__ void ring_body(const KParams& p, int64_t bid)
{
    const int rows = p.T < p.W ? p.T : p.W;
    const int g = (int)(bid / rows);
    const GMeta c = load_gmeta(p.meta, g, p.W);
    const int r = p.T - 1 - (int)(bid % rows);
    if (r < 0 || r < p.T - c.wg) return;
    const int slot = (int)(((int64_t)c.head0 + c.len0 + r) % c.wg);
    const float* ks = p.k + ((int64_t)r * p.G + g) * p.d;
    const float* vs = p.v + ((int64_t)r * p.G + g) * p.dv;
    float* kd = p.ring_k + ((int64_t)g * p.W + slot) * p.d;
    float* vd = p.ring_v + ((int64_t)g * p.W + slot) * p.dv;
    const float* kt = p.rope ? p.rope + (int64_t)r * p.d : nullptr;   // the ring holds turned keys
    for (int t = threadIdx.x; t < p.d / 4; t += blockDim.x)
        reinterpret_cast<float4*>(kd)[t] = rope4(ks, kt, 4 * t, p.d);
    for (int t = threadIdx.x; t < p.dv / 4; t += blockDim.x)
        reinterpret_cast<float4*>(vd)[t] = reinterpret_cast<const float4*>(vs)[t];
}

// len, head and nfar after T pushes (o1b_meta with k = T), from the
// call-start meta p.meta into the state's p.meta_out; one block of at least
// G (<= 64) threads.
__device__ __forceinline__ void meta_body(const KParams& p)
{
    const int g = threadIdx.x;
    if (g >= p.G) return;
    const GMeta c = load_gmeta(p.meta, g, p.W);
    const int64_t tot = (int64_t)c.len0 + p.T;
    uint32_t* mo = p.meta_out + 4 * g;
    if (tot <= c.wg) {
        mo[0] = (uint32_t)tot;
    } else {
        const int64_t ev = tot - c.wg;
        mo[0] = (uint32_t)c.wg;
        mo[1] = (uint32_t)((c.head0 + ev) % c.wg);
        mo[2] = (uint32_t)(c.nfar0 + ev);
    }
}

}  // namespace swl
