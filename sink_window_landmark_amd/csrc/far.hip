// Far-field kernels: eviction scores, the running max / mass scan, and the
// value accumulator.  cortiq-engine 0.8.51 src/gpu_wgpu/o1_batch.rs,
// o1b_far_e and o1b_far_commit, generalised from one sub-chunk to the S
// sub-chunks of a call: the score and value products of every sub-chunk run
// in parallel, and only the cheap per-landmark recurrences (M, Z, Theta) walk
// the sub-chunks in order.
#include "swl_internal.h"

namespace swl {

// ---------------------------------------------------------------------------
// far_score: L[s][gh*m+b][j] = scale * <q~_{gh,b}, key evicted by row j of
// sub-chunk s>, for the evicting rows j0 <= j < k_s; the other lanes hold
// -inf.  One block per (sub-chunk, group); the group's evicted keys of the
// sub-chunk are staged in LDS and every landmark row of the group reads them.
// ---------------------------------------------------------------------------
constexpr int FS_THREADS = 256;
constexpr int FS_J = 16;  // evicted rows per register tile

__global__ __launch_bounds__(FS_THREADS) void k_far_score(KParams p)
{
    extern __shared__ float lds[];
    const int s = blockIdx.x, g = blockIdx.y;
    const int r0 = s * SUB;
    const int ks = min(SUB, p.T - r0);
    const GMeta c = load_gmeta(p.meta, g, p.W);
    const SubMeta sm = sub_meta(c, r0);
    const int jlo = max(sm.j0, 0);
    const int d = p.d;
    const int hm = p.H * p.m;
    const int nhm = p.nh * p.m;
    float* ek = lds;  // [SUB][d]
    for (int e = threadIdx.x; e < SUB * d; e += FS_THREADS) {
        int j = e / d, t = e % d;
        float x = 0.f;
        if (j >= jlo && j < ks) x = key_row(p, c, g, c.len0 + r0 + j - c.wg)[t];
        ek[e] = x;
    }
    __syncthreads();
    float* L = p.E + ((int64_t)s * nhm + (int64_t)g * hm) * SUB;
    // work item: (landmark row hb, tile of FS_J evicted rows)
    const int ntile = SUB / FS_J;
    for (int w = threadIdx.x; w < hm * ntile; w += FS_THREADS) {
        const int hb = w / ntile, jt = (w % ntile) * FS_J;
        const float* qt = p.q_tilde + ((int64_t)g * hm + hb) * d;
        float acc[FS_J];
#pragma unroll
        for (int u = 0; u < FS_J; ++u) acc[u] = 0.f;
        for (int t = 0; t < d; t += 4) {
            float4 qv = *reinterpret_cast<const float4*>(qt + t);
#pragma unroll
            for (int u = 0; u < FS_J; ++u) {
                float4 kv = *reinterpret_cast<const float4*>(ek + (jt + u) * d + t);
                acc[u] += qv.x * kv.x + qv.y * kv.y + qv.z * kv.z + qv.w * kv.w;
            }
        }
#pragma unroll
        for (int u = 0; u < FS_J; ++u) {
            int j = jt + u;
            L[(int64_t)hb * SUB + j] = (j >= jlo && j < ks) ? acc[u] * p.scale : -INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// far_scan: one wave per (gh, b), lane j = chunk row j (as o1b_far_e), walking
// the sub-chunks in order.  Per sub-chunk: M' = max(M, max_j l_j); R = 1 if
// M' == M else exp(M - M') (an empty field at -inf gets R = 1 until its first
// eviction, which then rescales the zero mass by exp(-inf) = 0);
// E_j = exp(l_j - M') for evicting rows, else 0; P_j = R*Z + inclusive
// prefix of E (a wave scan in place of the pages' serial lane-0 loop);
// Z <- P_63; M <- M'.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

__device__ __forceinline__ float wave_incl_scan(float x, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        float y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

__global__ __launch_bounds__(256) void k_far_scan(KParams p)
{
    const int lane = threadIdx.x & 63;
    const int ghb = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nhm = p.nh * p.m;
    if (ghb >= nhm) return;
    const int gh = ghb / p.m, b = ghb % p.m, g = gh / p.H;
    const GMeta c = load_gmeta(p.meta, g, p.W);
    float M = p.mz[(int64_t)gh * 2 * p.m + b];
    float Z = p.mz[(int64_t)gh * 2 * p.m + p.m + b];
    float lnext = p.E[(int64_t)ghb * SUB + lane];
    for (int s = 0; s < p.S; ++s) {
        const float l = lnext;
        if (s + 1 < p.S) lnext = p.E[((int64_t)(s + 1) * nhm + ghb) * SUB + lane];
        const int r0 = s * SUB;
        const int ks = min(SUB, p.T - r0);
        const SubMeta sm = sub_meta(c, r0);
        const bool ev = lane >= sm.j0 && lane < ks;
        const float mx = wave_max(ev ? l : -INFINITY);
        const float Mn = fmaxf(M, mx);
        const float R = (Mn == M) ? 1.0f : expf(M - Mn);
        const float e = ev ? expf(l - Mn) : 0.0f;
        const float pf = R * Z + wave_incl_scan(e, lane);
        const int64_t at = ((int64_t)s * nhm + ghb) * SUB + lane;
        p.E[at] = e;
        p.P[at] = pf;
        if (lane == 0) {
            p.Ms[(int64_t)s * nhm + ghb] = Mn;
            p.Rs[(int64_t)s * nhm + ghb] = R;
        }
        Z = __shfl(pf, 63, 64);
        M = Mn;
    }
}

// ---------------------------------------------------------------------------
// dtheta: TH[s][gh*m+b][t] = sum_j E[s][gh*m+b][j] * v_evicted(s, j)[t], the
// value the sub-chunk adds to each landmark's accumulator (o1b_far_commit's
// sum over the evicted rows).  One block per (sub-chunk, query head).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_dtheta(KParams p)
{
    extern __shared__ float lds[];
    const int s = blockIdx.x, gh = blockIdx.y, g = gh / p.H;
    const int r0 = s * SUB;
    const int ks = min(SUB, p.T - r0);
    const GMeta c = load_gmeta(p.meta, g, p.W);
    const SubMeta sm = sub_meta(c, r0);
    const int jlo = max(sm.j0, 0);
    const int dv = p.dv, m = p.m;
    const int nhm = p.nh * m;
    float* vev = lds;               // [SUB][dv]
    float* eb = lds + SUB * dv;     // [m][SUB]
    for (int e = threadIdx.x; e < SUB * dv; e += 256) {
        int j = e / dv, t = e % dv;
        float x = 0.f;
        if (j >= jlo && j < ks) x = val_row(p, c, g, c.len0 + r0 + j - c.wg)[t];
        vev[e] = x;
    }
    const float* E = p.E + ((int64_t)s * nhm + (int64_t)gh * m) * SUB;
    for (int e = threadIdx.x; e < m * SUB; e += 256) eb[e] = E[e];
    __syncthreads();
    float* out = p.TH + ((int64_t)s * nhm + (int64_t)gh * m) * dv;
    const int nq = dv / 4;
    for (int w = threadIdx.x; w < m * nq; w += 256) {
        const int b = w / nq, t = (w % nq) * 4;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = jlo; j < ks; ++j) {
            const float ej = eb[b * SUB + j];
            const float4 vv = *reinterpret_cast<const float4*>(vev + j * dv + t);
            acc.x += ej * vv.x;
            acc.y += ej * vv.y;
            acc.z += ej * vv.z;
            acc.w += ej * vv.w;
        }
        *reinterpret_cast<float4*>(out + (int64_t)b * dv + t) = acc;
    }
}

// ---------------------------------------------------------------------------
// theta_scan: one thread per (gh, b, t), walking the sub-chunks in order:
// TH[s] <- Theta (the value before sub-chunk s, which the readout of s uses),
// Theta <- R_s Theta + dTheta_s.  With `commit` the final Theta, M and Z go
// to the state (o1b_far_commit: M <- M', Z <- P_{k-1}).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_theta_scan(KParams p, int commit)
{
    const int64_t nhm = (int64_t)p.nh * p.m;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= nhm * p.dv) return;
    const int64_t ghb = idx / p.dv;
    float th = p.theta[idx];
    float dnext = p.TH[idx];
    for (int s = 0; s < p.S; ++s) {
        const float dth = dnext;
        if (s + 1 < p.S) dnext = p.TH[(int64_t)(s + 1) * nhm * p.dv + idx];
        p.TH[(int64_t)s * nhm * p.dv + idx] = th;
        th = p.Rs[(int64_t)s * nhm + ghb] * th + dth;
    }
    if (commit) {
        p.theta[idx] = th;
        if (idx % p.dv == 0) {
            const int64_t gh = ghb / p.m, b = ghb % p.m;
            const int64_t last = (int64_t)(p.S - 1) * nhm + ghb;
            p.mz[gh * 2 * p.m + b] = p.Ms[last];
            p.mz[gh * 2 * p.m + p.m + b] = p.P[last * SUB + (SUB - 1)];
        }
    }
}

// ---------------------------------------------------------------------------
hipError_t launch_far_score(const KParams& p, hipStream_t st)
{
    size_t lds = sizeof(float) * SUB * p.d;
    hipLaunchKernelGGL(k_far_score, dim3(p.S, p.G), dim3(FS_THREADS), lds, st, p);
    return hipGetLastError();
}

hipError_t launch_far_scan(const KParams& p, hipStream_t st)
{
    int nhm = p.nh * p.m;
    hipLaunchKernelGGL(k_far_scan, dim3((nhm + 3) / 4), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_dtheta(const KParams& p, hipStream_t st)
{
    size_t lds = sizeof(float) * (SUB * p.dv + p.m * SUB);
    hipLaunchKernelGGL(k_dtheta, dim3(p.S, p.nh), dim3(256), lds, st, p);
    return hipGetLastError();
}

hipError_t launch_theta_scan(const KParams& p, bool commit, hipStream_t st)
{
    int64_t n = (int64_t)p.nh * p.m * p.dv;
    hipLaunchKernelGGL(k_theta_scan, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p,
                       commit ? 1 : 0);
    return hipGetLastError();
}

}  // namespace swl
