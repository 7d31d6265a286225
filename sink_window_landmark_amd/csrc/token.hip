// One-row decode: a sub-chunk of one row with commit (cortiq-engine 0.8.82
// src/gpu_metal/o1c.rs, encode_tok: near partials and the far part are
// independent, then a merge, then the commit), in two launches.
//
// k_tok_part: blocks of two kinds run side by side.
//   near (group g, split sp): keys sp*64 .. sp*64+63 of the row's keys
//     (the sinks, then the window after the push: logical x of the new ring
//     at slot (head' + x) mod w_g, the newest one being the row's own key),
//     for every head of the group: a partial (max, mass, value sum) in
//     base 2.
//   far (query head gh, landmark range fb): when the ring is full the row
//     evicts the key at slot head; every landmark b of the range folds it in
//     (l = scale <q~_b, k_e>, M' = max(M, l), R = 1 if M' == M else
//     e^{M-M'}, Z' = R Z + e^{l-M'}, Theta' = R Theta + e^{l-M'} v_e: o1b_far_e
//     and o1b_far_commit for one row) and writes M', Z', Theta' back.  Then
//     the far estimate of the range against M': u_b = sum_a e^{f_a-f_max}
//     mu[a][b] (>= 0 with rect), gain_b against the range's own exponent,
//     D = sum_b gain_b Z'_b and N = sum_b gain_b Theta'_b -- for a one-row
//     chunk, the chunk form's R Theta + cf v_e is exactly Theta'.
// k_tok_merge: one block per query head: the head's partials brought to one
//   exponent c = max of all partial maxima (the pages' c = max(c_near,
//   f_max + M'_b)), the far part dropped when its total mass is not >= 0,
//   out = (N + sum p v) / max(D + sum p, 1e-30); the first head of each
//   group then pushes the row into the ring (slot head when the ring is full,
//   else (head + len)) and advances meta.
#include "swl_internal.h"

namespace swl {

constexpr int TOK_KEYS = 64;    // keys per near block
constexpr int TOK_FB = 4;       // far blocks per query head (landmark ranges)
constexpr int TOK_BMAX = 16;    // landmarks per far block (m <= 64)
constexpr int TOK_THREADS = 256;
constexpr float TOK_LOG2E = 1.4426950408889634f;

int tok_splits(int ns, int W) { return (ns + W + TOK_KEYS - 1) / TOK_KEYS; }

// partial record: [0] max (base 2), [1] mass, [2 .. 2+dv) value sum
__host__ __device__ inline int64_t tok_rec(int dv) { return 2 + dv; }

size_t tok_part_floats(int G, int H, int dv, int ns, int W)
{
    return (size_t)G * tok_splits(ns, W) * H * tok_rec(dv) + (size_t)G * H * TOK_FB * tok_rec(dv);
}

struct TokRow {
    int full, slot, len1, head1, nfar1;
};

__device__ __forceinline__ TokRow tok_row(const GMeta& c)
{
    TokRow r;
    r.full = c.len0 >= c.wg;
    r.slot = r.full ? c.head0 : (c.head0 + c.len0) % c.wg;
    r.len1 = r.full ? c.wg : c.len0 + 1;
    r.head1 = r.full ? (c.head0 + 1) % c.wg : c.head0;
    r.nfar1 = c.nfar0 + (r.full ? 1 : 0);
    return r;
}

__device__ __forceinline__ float wsum(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

__device__ __forceinline__ float wmax(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

// Sum of x over groups of n consecutive lanes (n a power of two <= 64).
__device__ __forceinline__ float group_sum(float x, int n)
{
    for (int o = n >> 1; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// Every block first issues all of its global loads into LDS (one round
// trip), then computes from LDS.
__global__ __launch_bounds__(TOK_THREADS) void k_tok_part(KParams p, float* part, int nsplit)
{
    extern __shared__ float lds[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int d = p.d, dv = p.dv, H = p.H, m = p.m;
    const int nnear = p.G * nsplit;
    float* nearp = part;                                           // [G][nsplit][H][rec]
    float* farp = part + (int64_t)p.G * nsplit * H * tok_rec(dv);  // [nh][FB][rec]

    if ((int)blockIdx.x < nnear) {
        // ---------------- near partial ----------------
        const int g = blockIdx.x / nsplit, sp = blockIdx.x % nsplit;
        const GMeta c = load_gmeta(p.meta, g, p.W);
        const TokRow r = tok_row(c);
        const int n = p.ns + r.len1;
        const int k0 = sp * TOK_KEYS, k1 = min(n, k0 + TOK_KEYS);
        float* base = nearp + (int64_t)g * nsplit * H * tok_rec(dv);
        if (k0 >= k1) {
            for (int e = tid; e < H * tok_rec(dv); e += TOK_THREADS) {
                const int h = e / tok_rec(dv), f = e % tok_rec(dv);
                base[((int64_t)sp * H + h) * tok_rec(dv) + f] = f == 0 ? -INFINITY : 0.f;
            }
            return;
        }
        const int nk = k1 - k0;
        const int LDK = d + 4, LDV = dv + 4;
        float* Kl = lds;                      // [64][d+4]
        float* Vl = Kl + TOK_KEYS * LDK;      // [64][dv+4]
        float* Ql = Vl + TOK_KEYS * LDV;      // [H][d]
        float* Pl = Ql + H * d;               // [H][64] scores, then weights
        float* ST = Pl + H * TOK_KEYS;        // [H][2] max, mass
        for (int e = tid; e < TOK_KEYS * (d / 4); e += TOK_THREADS) {
            const int row = e / (d / 4), c4 = (e % (d / 4)) * 4;
            const int x = k0 + row;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (x < k1) {
                const float *kp, *vp;
                if (x < p.ns) {
                    kp = p.sink_k + ((int64_t)g * p.ns + x) * d;
                    vp = p.sink_v + ((int64_t)g * p.ns + x) * dv;
                } else if (x - p.ns == r.len1 - 1) {   // the row's own key
                    kp = p.k + (int64_t)g * d;
                    vp = p.v + (int64_t)g * dv;
                } else {
                    const int slot = (r.head1 + x - p.ns) % c.wg;
                    kp = p.ring_k + ((int64_t)g * p.W + slot) * d;
                    vp = p.ring_v + ((int64_t)g * p.W + slot) * dv;
                }
                kx = *reinterpret_cast<const float4*>(kp + c4);
                vx = *reinterpret_cast<const float4*>(vp + c4);
            }
            *reinterpret_cast<float4*>(Kl + row * LDK + c4) = kx;
            *reinterpret_cast<float4*>(Vl + row * LDV + c4) = vx;
        }
        const float qs = p.scale * TOK_LOG2E;
        for (int e = tid; e < H * d; e += TOK_THREADS) Ql[e] = p.q[(int64_t)g * H * d + e] * qs;
        __syncthreads();
        // scores: thread per (head, key)
        for (int e = tid; e < H * TOK_KEYS; e += TOK_THREADS) {
            const int h = e / TOK_KEYS, j = e % TOK_KEYS;
            float acc = -INFINITY;
            if (j < nk) {
                const float* kr = Kl + j * LDK;
                const float* qr = Ql + h * d;
                acc = 0.f;
#pragma unroll 8
                for (int t = 0; t < d; t += 4) {
                    const float4 a = *reinterpret_cast<const float4*>(kr + t);
                    const float4 b = *reinterpret_cast<const float4*>(qr + t);
                    acc += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
                }
            }
            Pl[e] = acc;
        }
        __syncthreads();
        // per head: max, weights, mass (a wave per head, lane = key)
        for (int h = wave; h < H; h += TOK_THREADS / 64) {
            const float sc = Pl[h * TOK_KEYS + lane];
            const float mx = wmax(sc);
            const float pv = lane < nk ? exp2f(sc - mx) : 0.f;
            const float l = wsum(pv);
            Pl[h * TOK_KEYS + lane] = pv;
            if (lane == 0) {
                ST[2 * h] = mx;
                ST[2 * h + 1] = l;
            }
        }
        __syncthreads();
        // value sums: thread per (head, value column)
        for (int e = tid; e < H * dv; e += TOK_THREADS) {
            const int h = e / dv, t = e % dv;
            const float* pr = Pl + h * TOK_KEYS;
            float acc = 0.f;
#pragma unroll 8
            for (int j = 0; j < nk; ++j) acc += pr[j] * Vl[j * LDV + t];
            float* rec = base + ((int64_t)sp * H + h) * tok_rec(dv);
            rec[2 + t] = acc;
            if (t == 0) {
                rec[0] = ST[2 * h];
                rec[1] = ST[2 * h + 1];
            }
        }
        return;
    }

    // ---------------- far partial ----------------
    const int fbk = blockIdx.x - nnear;
    const int gh = fbk / TOK_FB, fb = fbk % TOK_FB;
    const int g = gh / H;
    const GMeta c = load_gmeta(p.meta, g, p.W);
    const TokRow r = tok_row(c);
    float* rec = farp + ((int64_t)gh * TOK_FB + fb) * tok_rec(dv);
    const int per = (m + TOK_FB - 1) / TOK_FB;   // <= TOK_BMAX
    const int b0 = fb * per, b1 = min(m, b0 + per), nb = b1 - b0;
    if (r.nfar1 == 0 || nb <= 0) {
        for (int t = tid; t < tok_rec(dv); t += TOK_THREADS) rec[t] = t == 0 ? -INFINITY : 0.f;
        return;
    }
    const int LDT = d + 4;
    float* Ql = lds;                  // [d]
    float* KE = Ql + d;               // [d]       evicted key
    float* VE = KE + d;               // [dv]      evicted value
    float* KT = VE + dv;              // [m][d+4]  landmark keys
    float* QT = KT + m * LDT;         // [16][d+4] this range's landmark queries
    float* TH = QT + TOK_BMAX * LDT;  // [16][dv]  this range's accumulators
    float* MU = TH + TOK_BMAX * dv;   // [m][16]   mu[a][b0 + j]
    float* EA = MU + m * TOK_BMAX;    // [64]      f_a, then e_a
    float* MB = EA + 64;              // [16]      M'
    float* RB = MB + 16;              // [16]      R
    float* XB = RB + 16;              // [16]      exp(l - M')
    float* ZB = XB + 16;              // [16]      Z'
    float* GB = ZB + 16;              // [16]      gains
    float* RED = GB + 16;             // [4]
    float* mz = p.mz + (int64_t)gh * 2 * m;
    const float* ring_k_e = p.ring_k + ((int64_t)g * p.W + c.head0) * d;
    const float* ring_v_e = p.ring_v + ((int64_t)g * p.W + c.head0) * dv;
    for (int t = tid; t < d; t += TOK_THREADS) {
        Ql[t] = p.q[(int64_t)gh * d + t];
        KE[t] = r.full ? ring_k_e[t] : 0.f;
    }
    for (int t = tid; t < dv; t += TOK_THREADS) VE[t] = r.full ? ring_v_e[t] : 0.f;
    for (int e = tid; e < m * (d / 4); e += TOK_THREADS) {
        const int a = e / (d / 4), c4 = (e % (d / 4)) * 4;
        *reinterpret_cast<float4*>(KT + a * LDT + c4) =
            *reinterpret_cast<const float4*>(p.k_tilde + ((int64_t)g * m + a) * d + c4);
    }
    for (int e = tid; e < nb * (d / 4); e += TOK_THREADS) {
        const int j = e / (d / 4), c4 = (e % (d / 4)) * 4;
        *reinterpret_cast<float4*>(QT + j * LDT + c4) =
            *reinterpret_cast<const float4*>(p.q_tilde + ((int64_t)gh * m + b0 + j) * d + c4);
    }
    const float* th_g = p.theta + ((int64_t)gh * m + b0) * dv;
    for (int e = tid; e < nb * (dv / 4); e += TOK_THREADS)
        *reinterpret_cast<float4*>(TH + e * 4) = *reinterpret_cast<const float4*>(th_g + e * 4);
    for (int e = tid; e < m * nb; e += TOK_THREADS) {
        const int a = e / nb, j = e % nb;
        MU[a * TOK_BMAX + j] = p.mu[((int64_t)gh * m + a) * m + b0 + j];
    }
    __syncthreads();
    // f_a (base 2) for every landmark: 4 lanes per landmark
    for (int e = tid; e < 64 * 4; e += TOK_THREADS) {
        const int a = e >> 2, qq = e & 3;
        float acc = 0.f;
        if (a < m) {
            const float* kr = KT + a * LDT;
            for (int t = qq * 4; t < d; t += 16) {
                const float4 x = *reinterpret_cast<const float4*>(kr + t);
                acc += x.x * Ql[t] + x.y * Ql[t + 1] + x.z * Ql[t + 2] + x.w * Ql[t + 3];
            }
        }
        acc = group_sum(acc, 4);
        if (qq == 0 && a < m) EA[a] = acc * p.scale * TOK_LOG2E;
    }
    // the evicted key folded into each landmark of the range: 16 lanes each
    {
        const int j = tid >> 4, qq = tid & 15;   // 16 landmarks x 16 lanes
        float acc = 0.f;
        if (j < nb && r.full) {
            const float* qr = QT + j * LDT;
            for (int t = qq * 4; t < d; t += 64) {
                const float4 y = *reinterpret_cast<const float4*>(qr + t);
                acc += y.x * KE[t] + y.y * KE[t + 1] + y.z * KE[t + 2] + y.w * KE[t + 3];
            }
        }
        acc = group_sum(acc, 16);
        if (qq == 0 && j < nb) {
            const int b = b0 + j;
            const float Mo = mz[b], Zo = mz[m + b];
            float Mn = Mo, R = 1.f, x = 0.f, Zn = Zo;
            if (r.full) {
                const float l = acc * p.scale;
                Mn = fmaxf(Mo, l);
                R = (Mn == Mo) ? 1.f : expf(Mo - Mn);
                x = expf(l - Mn);
                Zn = Zo * R + x;
                mz[b] = Mn;
                mz[m + b] = Zn;
            }
            MB[j] = Mn;
            RB[j] = R;
            XB[j] = x;
            ZB[j] = Zn;
        }
    }
    __syncthreads();
    if (wave == 0) {
        const float f = lane < m ? EA[lane] : -INFINITY;
        const float fmax = wmax(f);
        if (lane < m) EA[lane] = exp2f(f - fmax);
        if (lane == 0) RED[0] = fmax;
    } else if (wave == 1) {
        const float mm = wmax(lane < nb ? MB[lane] : -INFINITY);
        if (lane == 0) RED[1] = mm;
    }
    __syncthreads();
    const float fmax = RED[0];
    const float cl = fmax + RED[1] * TOK_LOG2E;   // the range's exponent, base 2
    // u_b = sum_a e_a mu[a][b] and the gains: 16 lanes per landmark
    {
        const int j = tid >> 4, qq = tid & 15;
        float u = 0.f;
        if (j < nb)
            for (int a = qq; a < m; a += 16) u += EA[a] * MU[a * TOK_BMAX + j];
        u = group_sum(u, 16);
        if (qq == 0 && j < nb) {
            if (p.rect) u = fmaxf(u, 0.f);
            GB[j] = u * exp2f(fmax + MB[j] * TOK_LOG2E - cl);
        }
    }
    __syncthreads();
    if (wave == 0) {
        const float dd = wsum(lane < nb ? GB[lane] * ZB[lane] : 0.f);
        if (lane == 0) {
            rec[0] = cl;
            rec[1] = dd;
        }
    }
    // Theta' = R Theta + x v_e (written back) and N = sum_b gain_b Theta'_b
    float* th = p.theta + ((int64_t)gh * m + b0) * dv;
    for (int t = tid; t < dv; t += TOK_THREADS) {
        float acc = 0.f;
        for (int j = 0; j < nb; ++j) {
            float x = TH[j * dv + t];
            if (r.full) {
                x = x * RB[j] + XB[j] * VE[t];
                th[(int64_t)j * dv + t] = x;
            }
            acc += GB[j] * x;
        }
        rec[2 + t] = acc;
    }
}

// One block per query head: the head's partials to one exponent, the far
// part dropped when its total mass is not >= 0, out.  The first head of a
// group also pushes the row into the ring and advances meta (no other block
// of this kernel reads them).
__global__ __launch_bounds__(TOK_THREADS) void k_tok_merge(KParams p, const float* part, int nsplit)
{
    extern __shared__ float lds[];
    const int gh = blockIdx.x, g = gh / p.H, h = gh % p.H;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int H = p.H, dv = p.dv;
    const int64_t rl = tok_rec(dv);
    const float* nearp = part + (int64_t)g * nsplit * H * rl + (int64_t)h * rl;   // stride H*rl
    const float* farp = part + (int64_t)p.G * nsplit * H * rl + (int64_t)gh * TOK_FB * rl;
    const int nrec = nsplit + TOK_FB;
    float* WS = lds;              // [nrec] weights (near splits, then far ranges)
    float* ACC = WS + nrec;       // [TOK_THREADS / dv >= 1][dv] partial sums
    float* RED = ACC + 2 * dv;    // [4]
    const bool farok = farp[0] != -INFINITY;   // far records hold -inf when the far field is empty
    if (wave == 0) {
        float cmax = -INFINITY;
        for (int k = lane; k < nrec; k += 64) {
            const float* rc = k < nsplit ? nearp + (int64_t)k * H * rl : farp + (int64_t)(k - nsplit) * rl;
            if (k < nsplit || farok) cmax = fmaxf(cmax, rc[0]);
        }
        cmax = wmax(cmax);
        float den = 0.f, dfar = 0.f;
        for (int k = lane; k < nrec; k += 64) {
            const float* rc = k < nsplit ? nearp + (int64_t)k * H * rl : farp + (int64_t)(k - nsplit) * rl;
            float w = 0.f;
            if (k < nsplit || farok) w = exp2f(rc[0] - cmax);
            if (k < nsplit) den += rc[1] * w;
            else dfar += rc[1] * w;
            WS[k] = w;
        }
        den = wsum(den);
        dfar = wsum(dfar);
        const bool have = farok && dfar >= 0.f;
        if (lane == 0) {
            RED[0] = 1.f / fmaxf(den + (have ? dfar : 0.f), 1e-30f);
            RED[1] = have ? 1.f : 0.f;
        }
    }
    __syncthreads();
    const float inv = RED[0];
    const bool have = RED[1] > 0.5f;
    // two halves of the records over value columns; each thread issues all
    // of its loads before it sums
    const int halves = dv <= TOK_THREADS / 2 ? 2 : 1;
    const int t = tid % (TOK_THREADS / halves), hb = tid / (TOK_THREADS / halves);
    const int kend = have ? nrec : nsplit;
    const int per = (kend + halves - 1) / halves;
    const int ka = hb * per, kb = min(kend, ka + per);
    if (t < dv) {
        float acc = 0.f;
        for (int k0 = ka; k0 < kb; k0 += 8) {
            float x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int k = k0 + u;
                const float* rc = k < nsplit ? nearp + (int64_t)k * H * rl : farp + (int64_t)(k - nsplit) * rl;
                x[u] = k < kb ? rc[2 + t] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (k0 + u < kb) acc += x[u] * WS[k0 + u];
        }
        ACC[hb * dv + t] = acc;
    }
    __syncthreads();
    float* orow = p.out + (int64_t)gh * dv;
    for (int c2 = tid; c2 < dv; c2 += TOK_THREADS)
        orow[c2] = (ACC[c2] + (halves == 2 ? ACC[dv + c2] : 0.f)) * inv;
    if (h == 0) {
        // commit: ring push and meta (every reader of the ring and meta of
        // this group ran in the previous kernel)
        const GMeta c = load_gmeta(p.meta, g, p.W);
        const TokRow r = tok_row(c);
        __syncthreads();   // all threads have read meta before thread 0 writes it
        float* kd = p.ring_k + ((int64_t)g * p.W + r.slot) * p.d;
        float* vd = p.ring_v + ((int64_t)g * p.W + r.slot) * dv;
        for (int e = tid; e < p.d; e += TOK_THREADS) kd[e] = p.k[(int64_t)g * p.d + e];
        for (int e = tid; e < dv; e += TOK_THREADS) vd[e] = p.v[(int64_t)g * dv + e];
        if (tid == 0) {
            p.meta[4 * g + 0] = (uint32_t)r.len1;
            p.meta[4 * g + 1] = (uint32_t)r.head1;
            p.meta[4 * g + 2] = (uint32_t)r.nfar1;
        }
    }
}

hipError_t launch_token(const KParams& p, float* part, hipStream_t st)
{
    const int nsplit = tok_splits(p.ns, p.W);
    const size_t lds_near = sizeof(float) * ((size_t)TOK_KEYS * (p.d + 4) + (size_t)TOK_KEYS * (p.dv + 4) +
                                             (size_t)p.H * p.d + (size_t)p.H * TOK_KEYS + 2 * p.H);
    const size_t lds_far = sizeof(float) * ((size_t)2 * p.d + p.dv + (size_t)p.m * (p.d + 4) +
                                            (size_t)TOK_BMAX * (p.d + 4) + (size_t)TOK_BMAX * p.dv +
                                            (size_t)p.m * TOK_BMAX + 64 + 5 * 16 + 4);
    const size_t lds = lds_near > lds_far ? lds_near : lds_far;
    const int blocks = p.G * nsplit + p.nh * TOK_FB;
    // dynamic LDS beyond 64 KiB has to be allowed explicitly
    static size_t lds_allowed = 64 * 1024;
    if (lds > lds_allowed) {
        const hipError_t e = hipFuncSetAttribute((const void*)k_tok_part,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        lds_allowed = lds;
    }
    hipLaunchKernelGGL(k_tok_part, dim3(blocks), dim3(TOK_THREADS), lds, st, p, part, nsplit);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds_merge = sizeof(float) * ((size_t)nsplit + TOK_FB + 2 * p.dv + 4);
    hipLaunchKernelGGL(k_tok_merge, dim3(p.nh), dim3(TOK_THREADS), lds_merge, st, p,
                       (const float*)part, nsplit);
    return hipGetLastError();
}

}  // namespace swl
