// Device bodies of the small stages of a call -- the far accumulator scan,
// the ring commit and the meta update -- so that one launch can run them
// beside another stage: each block takes its role from its index, and no
// block waits on another.  cortiq-engine 0.8.51 src/gpu_wgpu/o1_batch.rs,
// o1b_far_commit, o1b_ring_commit and o1b_meta.
#pragma once

#include "swl_internal.h"
#include "lanes.h"

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

// ---------------------------------------------------------------------------
// mz_scan: one thread per landmark row (gh, b), walking the sub-chunks in
// order on scalars: M'_s, R_s, the factor fac_s = exp(mx_s - M'_s) that
// brings the sub-chunk's E to the post-sub-chunk max, and the incoming mass
// Z_{s-1} (into TZ[s]), with Z_s = R_s Z_{s-1} + zl_s fac_s, and the final
// mass into TZ[S].  Reads the local (mx, zl) that far_score left in Ms/Rs
// and replaces them with M'_s and R_s.
// ---------------------------------------------------------------------------
// (M, Z) of a run of sub-chunks: the max and the mass against it; a run
// with no evictions is (-inf, 0).  Runs a then b combine to the pair of the
// concatenation: the online-softmax merge, an associative operation.
struct MZ {
    float M, Z;
};
__device__ __forceinline__ MZ mz_merge(MZ a, MZ b)
{
    const float M = fmaxf(a.M, b.M);
    const float za = a.M == -INFINITY ? 0.f : a.Z * expf(a.M - M);
    const float zb = b.M == -INFINITY ? 0.f : b.Z * expf(b.M - M);
    return {M, za + zb};
}

// One wave per landmark row; lane l takes sub-chunks per l .. per l + per -
// 1, per = ceil(S / 64) <= MZ_PER (MZ_PER = PASS_SUBS / 64, so S <=
// PASS_SUBS):
// the merge of each lane's run, an exclusive scan of the runs over the wave,
// then every lane applies the recurrence above to its own sub-chunks from
// the state before them (so M'_s and R_s are exactly the serial ones and Z
// differs from the serial sum only in rounding order).
constexpr int MZ_PER = PASS_SUBS / 64;

// The largest |value| of share `bi` of `nb` equal shares of group g's value
// rows -- the sinks, the window at the call's start and the call's rows --
// into p.vmax[g][bi], by a block of NTHR threads (`red`: NTHR / 64 floats
// of LDS).  The value products of the call (key tiles, far readout) scale
// their fp16 splits by the group's maximum (value_exp).  The block's loads
// stay in flight U steps at a time.
template <int D, int NTHR>
__device__ __forceinline__ void value_max_share(const KParams& p, const GMeta& c, int g, int bi, int nb, float* red)
{
    constexpr int LPR = D / 4 < 64 ? D / 4 : 64;   // lanes per row (d <= 256: one float4 each)
    constexpr int RPB = NTHR / LPR;                 // rows per step
    constexpr int U = 4;                            // steps in flight
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n = (int64_t)p.ns + c.len0 + p.T;
    const int r_lo = (int)(n * bi / nb), r_hi = (int)(n * (bi + 1) / nb);
    const int li = tid % LPR, rb = tid / LPR;
    float mx = 0.f;
    for (int r0 = r_lo + rb; r0 < r_hi; r0 += U * RPB) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = min(r0 + u * RPB, r_hi - 1);   // clamped: repeats a row of the share
            const float* row = r < p.ns ? p.sink_v + ((int64_t)g * p.ns + r) * D : val_row(p, c, g, r - p.ns);
            v[u] = *reinterpret_cast<const float4*>(row + 4 * li);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
    }
    mx = wmax(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    if (tid == 0) {
        float b = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NTHR / 64; ++w2) b = fmaxf(b, red[w2]);
        p.vmax[(int64_t)g * VM_SLOTS + bi] = b;
    }
}

// The scan of one landmark row (gh, b) by one wave: LD(s) gives the local
// (mx, zl) of sub-chunk s < p.S, ST(s, M', R, Z before, fac) takes the
// results, and the mass after the last sub-chunk goes to ST(p.S, ...).
template <class LD, class ST>
__device__ __forceinline__ void mz_scan_row(const KParams& p, int64_t ghb, int lane, LD ld, ST st)
{
    const int64_t gh = ghb / p.m, b = ghb % p.m;
    const int per = (p.S + 63) / 64;   // (uniform)
    float mx[MZ_PER], zl[MZ_PER];
#pragma unroll
    for (int k = 0; k < MZ_PER; ++k) {
        const int s = min(per * lane + k, p.S - 1);
        const float2 x = ld(s);
        mx[k] = x.x;
        zl[k] = x.y;
        if (k >= per || per * lane + k >= p.S) mx[k] = -INFINITY;   // past the lane's run or the last sub-chunk: empty
    }
    MZ run = {-INFINITY, 0.f};
#pragma unroll
    for (int k = 0; k < MZ_PER; ++k)
        if (k < per) run = mz_merge(run, MZ{mx[k], zl[k]});
    // inclusive scan over the lanes, then shift to the exclusive prefix
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const MZ o = {__shfl_up(run.M, d, 64), __shfl_up(run.Z, d, 64)};
        if (lane >= d) run = mz_merge(o, run);
    }
    MZ pre = {__shfl_up(run.M, 1, 64), __shfl_up(run.Z, 1, 64)};
    if (lane == 0) pre = {-INFINITY, 0.f};
    // the committed state before the call, then this lane's sub-chunks
    const MZ s0 = mz_merge(MZ{p.mz[gh * 2 * p.m + b], p.mz[gh * 2 * p.m + p.m + b]}, pre);
    float M = s0.M, Z = s0.Z;
#pragma unroll
    for (int k = 0; k < MZ_PER; ++k) {
        const int s = per * lane + k;
        if (k < per && s < p.S) {
            const float Mn = fmaxf(M, mx[k]);
            const float R = (Mn == M) ? 1.0f : expf(M - Mn);
            const float fac = mx[k] == -INFINITY ? 0.f : expf(mx[k] - Mn);
            st(s, Mn, R, Z, fac);
            Z = R * Z + zl[k] * fac;
            M = Mn;
            // the mass after the last sub-chunk, which a commit stores: a call
            // that resumes from the committed state then carries this value
            if (s == p.S - 1) st(p.S, 0.f, 0.f, Z, 0.f);
        }
    }
}

// Blocks of 256 threads the far scan takes beside other work: a wave per
// landmark row, straight from and to the planes.
__host__ __device__ inline int64_t far_scan_blocks(const KParams& p)
{
    return ((int64_t)p.nh * p.m + 3) / 4;
}

__device__ __forceinline__ void mz_scan_body(const KParams& p, int64_t bid)
{
    const int64_t nhm = (int64_t)p.nh * p.m;
    const int lane = threadIdx.x & 63;
    const int64_t ghb = bid * 4 + (threadIdx.x >> 6);
    if (ghb >= nhm) return;   // (uniform over the wave)
    mz_scan_row(
        p, ghb, lane,
        [&](int s) {
            const int64_t at = (int64_t)s * nhm + ghb;
            return make_float2(p.Ms[at], p.Rs[at]);
        },
        [&](int s, float Mn, float R, float Z, float fac) {
            const int64_t at = (int64_t)s * nhm + ghb;
            if (s < p.S) {
                p.Ms[at] = Mn;
                p.Rs[at] = R;
                p.FAC[at] = fac;
            }
            p.TZ[at] = Z;
        });
}

// theta_scan, block `bid` of theta_blocks(p): one thread per (gh, b, t),
// walking the sub-chunks in order: TH[s] <- Theta (the value before
// sub-chunk s, which the readout of s uses), Theta <- R_s Theta +
// fac_s dTheta_s (far_score's increment is against the sub-chunk's own max;
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

// Ring commit, block `bid` of ring_blocks(p) (any block size): chunk row r of
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
    // the key's float4s, then the value's, over the block's threads
    for (int t = threadIdx.x; t < p.d / 4 + p.dv / 4; t += blockDim.x) {
        if (t < p.d / 4) reinterpret_cast<float4*>(kd)[t] = rope4(ks, kt, 4 * t, p.d);
        else reinterpret_cast<float4*>(vd)[t - p.d / 4] = reinterpret_cast<const float4*>(vs)[t - p.d / 4];
    }
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
