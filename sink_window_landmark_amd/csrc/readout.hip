// Far readout of a call, merged with the near part.
//
// cortiq-engine 0.8.51 src/gpu_wgpu/o1_batch.rs, o1b_attend (its far half):
// for each row i of a sub-chunk whose far field is not empty,
//   f_a = scale <q_i, k~_a>, u_b = sum_a exp(f_a - f_max) mu[a][b]
//   (clamped at 0 with rect), c = max(c_near, max_b f_max + M'_b),
//   gain_b = u_b exp(f_max + M'_b - c), D_far = sum_b gain_b P_bi,
//   cf_j = sum_b gain_b E_bj for the in-chunk evicted rows j0 <= j <= i,
//   N_far = sum_b gain_b R_b Theta_b + sum_j cf_j v_evicted(j);
// a D_far that is not >= 0 drops N_far and D_far.  The near part arrives
// as the normalised near output o (already in `out`) with its max c_near
// and mass l; it enters as l exp(c_near - c) (o, 1), so
//   out = (N_far + l e^{c_near-c} o) / max(D_far + l e^{c_near-c}, 1e-30).
// Rows whose far field is empty keep the near output unchanged (c = c_near
// and the mass is at least 1, as in the pages' kernel).
// One block per (sub-chunk, query head).
#include "swl_internal.h"

namespace swl {

constexpr int RO_THREADS = 256;

struct RoLayout {
    int a, f, mucf, gn, eb, rw, ms, rs, total;  // float offsets into LDS
};

__host__ __device__ inline RoLayout ro_layout(int d, int dv, int m)
{
    RoLayout L;
    int regA = SUB * d + m * d;
    int regF = m * dv + SUB * dv;
    L.a = 0;
    L.f = (regA > regF ? regA : regF);
    L.mucf = L.f + SUB * m;
    int mucf = m * m > SUB * SUB ? m * m : SUB * SUB;
    L.gn = L.mucf + mucf;
    L.eb = L.gn + SUB * m;
    L.rw = L.eb + m * SUB;
    L.ms = L.rw + SUB * 4;
    L.rs = L.ms + m;
    L.total = L.rs + m;
    return L;
}

__global__ __launch_bounds__(RO_THREADS) void k_readout(KParams p)
{
    extern __shared__ float lds[];
    const int s = blockIdx.x, gh = blockIdx.y, g = gh / p.H;
    const int tid = threadIdx.x;
    const int r0 = s * SUB;
    const int ks = min(SUB, p.T - r0);
    const GMeta c = load_gmeta(p.meta, g, p.W);
    const SubMeta sm = sub_meta(c, r0);
    const int jlo = max(sm.j0, 0);
    // first row with a non-empty far field
    const int ifar = sm.nfar0 > 0 ? 0 : jlo;
    if (ifar >= ks) return;
    const int d = p.d, dv = p.dv, m = p.m;
    const int64_t nhm = (int64_t)p.nh * m;
    const int64_t ghm0 = (int64_t)s * nhm + (int64_t)gh * m;  // row of (s, gh, b=0) in Ms/Rs
    const RoLayout L = ro_layout(d, dv, m);
    float* Qs = lds + L.a;            // [SUB][d]
    float* Kt = lds + L.a + SUB * d;  // [m][d]
    float* TH = lds + L.a;            // [m][dv]     (after Qs/Kt are done)
    float* VE = lds + L.a + m * dv;   // [SUB][dv]
    float* F = lds + L.f;             // [SUB][m]
    float* MU = lds + L.mucf;         // [m][m]
    float* CF = lds + L.mucf;         // [SUB][SUB]  (after MU is done)
    float* GN = lds + L.gn;           // [SUB][m]
    float* EB = lds + L.eb;           // [m][SUB]
    float* RW = lds + L.rw;           // [SUB][4]: c, near weight, D_far, have
    float* MS = lds + L.ms;           // [m]
    float* RS = lds + L.rs;           // [m]

    // phase A: f = scale q k~^T
    for (int e = tid; e < ks * d; e += RO_THREADS) {
        int i = e / d, t = e % d;
        Qs[e] = p.q[((int64_t)(r0 + i) * p.nh + gh) * d + t];
    }
    for (int e = tid; e < m * d; e += RO_THREADS) Kt[e] = p.k_tilde[(int64_t)g * m * d + e];
    for (int e = tid; e < m; e += RO_THREADS) {
        MS[e] = p.Ms[ghm0 + e];
        RS[e] = p.Rs[ghm0 + e];
    }
    __syncthreads();
    for (int w = tid; w < ks * m; w += RO_THREADS) {
        const int i = w / m, a = w % m;
        const float* qr = Qs + i * d;
        const float* kr = Kt + a * d;
        float acc = 0.f;
        for (int t = 0; t < d; t += 4) {
            const float4 x = *reinterpret_cast<const float4*>(qr + t);
            const float4 y = *reinterpret_cast<const float4*>(kr + t);
            acc += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
        }
        F[i * m + a] = acc * p.scale;
    }
    for (int e = tid; e < m * m; e += RO_THREADS) MU[e] = p.mu[(int64_t)gh * m * m + e];
    __syncthreads();
    // phase B: f_max and e_a = exp(f_a - f_max), per row
    if (tid < ks) {
        float* fr = F + tid * m;
        float fmax = -INFINITY;
        for (int a = 0; a < m; ++a) fmax = fmaxf(fmax, fr[a]);
        for (int a = 0; a < m; ++a) fr[a] = expf(fr[a] - fmax);
        RW[tid * 4 + 0] = fmax;
    }
    __syncthreads();
    // phase C: u_b = sum_a e_a mu[a][b]
    for (int w = tid; w < ks * m; w += RO_THREADS) {
        const int i = w / m, b = w % m;
        const float* er = F + i * m;
        float u = 0.f;
        for (int a = 0; a < m; ++a) u += er[a] * MU[a * m + b];
        if (p.rect) u = fmaxf(u, 0.f);
        GN[i * m + b] = u;
    }
    __syncthreads();
    // phase D: common exponent, gains and far mass, per row
    if (tid < ks) {
        const int i = tid;
        const int farl = sm.nfar0 + (i >= sm.j0 ? i - sm.j0 + 1 : 0);
        float cexp = 0.f, wn = 0.f, dfar = 0.f, have = 0.f;
        if (farl > 0) {
            const float fmax = RW[i * 4 + 0];
            const float* ns = p.NS + ((int64_t)(r0 + i) * p.nh + gh) * 2;
            const float cn = ns[0], ln = ns[1];
            float cc = cn;
            for (int b = 0; b < m; ++b) cc = fmaxf(cc, fmax + MS[b]);
            float* gr = GN + i * m;
            const float* P = p.P + ghm0 * SUB;
            for (int b = 0; b < m; ++b) {
                const float gain = gr[b] * expf(fmax + MS[b] - cc);
                gr[b] = gain;
                dfar += gain * P[(int64_t)b * SUB + i];
            }
            if (dfar >= 0.f) have = 1.f;
            else dfar = 0.f;
            cexp = cc;
            wn = ln * expf(cn - cc);
        }
        RW[i * 4 + 0] = cexp;
        RW[i * 4 + 1] = wn;
        RW[i * 4 + 2] = dfar;
        RW[i * 4 + 3] = have;
    }
    for (int e = tid; e < m * SUB; e += RO_THREADS) EB[e] = p.E[ghm0 * SUB + e];
    __syncthreads();
    // phase E: in-chunk coefficients cf_ij = sum_b gain_ib E_bj, j0 <= j <= i
    for (int w = tid; w < ks * SUB; w += RO_THREADS) {
        const int i = w / SUB, j = w % SUB;
        float cf = 0.f;
        if (RW[i * 4 + 3] > 0.5f && j >= jlo && j <= i) {
            const float* gr = GN + i * m;
            for (int b = 0; b < m; ++b) cf += gr[b] * EB[b * SUB + j];
        }
        CF[i * SUB + j] = cf;
    }
    // Theta before this sub-chunk and the evicted values
    const float* thp = p.theta_prev + (int64_t)s * p.theta_prev_stride + (int64_t)gh * m * dv;
    for (int e = tid; e < m * dv; e += RO_THREADS) TH[e] = thp[e];
    for (int e = tid; e < SUB * dv; e += RO_THREADS) {
        const int j = e / dv, t = e % dv;
        float x = 0.f;
        if (j >= jlo && j < ks) x = val_row(p, c, g, c.len0 + r0 + j - c.wg)[t];
        VE[e] = x;
    }
    __syncthreads();
    // phase F: N_far and the merge with the near output
    const int nq = dv / 4;
    for (int w = tid; w < ks * nq; w += RO_THREADS) {
        const int i = w / nq, t = (w % nq) * 4;
        const int farl = sm.nfar0 + (i >= sm.j0 ? i - sm.j0 + 1 : 0);
        if (farl <= 0) continue;
        const bool have = RW[i * 4 + 3] > 0.5f;
        float4 nf = make_float4(0.f, 0.f, 0.f, 0.f);
        if (have) {
            const float* gr = GN + i * m;
            for (int b = 0; b < m; ++b) {
                const float gb = gr[b] * RS[b];
                const float4 th = *reinterpret_cast<const float4*>(TH + b * dv + t);
                nf.x += gb * th.x;
                nf.y += gb * th.y;
                nf.z += gb * th.z;
                nf.w += gb * th.w;
            }
            const float* cr = CF + i * SUB;
            for (int j = jlo; j <= i; ++j) {
                const float cj = cr[j];
                const float4 vv = *reinterpret_cast<const float4*>(VE + j * dv + t);
                nf.x += cj * vv.x;
                nf.y += cj * vv.y;
                nf.z += cj * vv.z;
                nf.w += cj * vv.w;
            }
        }
        const float wn = RW[i * 4 + 1];
        const float den = fmaxf((have ? RW[i * 4 + 2] : 0.f) + wn, 1e-30f);
        float* orow = p.out + ((int64_t)(r0 + i) * p.nh + gh) * dv + t;
        const float4 o = *reinterpret_cast<const float4*>(orow);
        float4 r;
        r.x = (nf.x + wn * o.x) / den;
        r.y = (nf.y + wn * o.y) / den;
        r.z = (nf.z + wn * o.z) / den;
        r.w = (nf.w + wn * o.w) / den;
        *reinterpret_cast<float4*>(orow) = r;
    }
}

hipError_t launch_readout(const KParams& p, hipStream_t st)
{
    const RoLayout L = ro_layout(p.d, p.dv, p.m);
    const size_t lds = sizeof(float) * (size_t)L.total;
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute((const void*)k_readout, hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024);
        attr_set = true;
    }
    hipLaunchKernelGGL(k_readout, dim3(p.S, p.nh), dim3(RO_THREADS), lds, st, p);
    return hipGetLastError();
}

size_t readout_lds_bytes(int d, int dv, int m)
{
    return sizeof(float) * (size_t)ro_layout(d, dv, m).total;
}

}  // namespace swl
