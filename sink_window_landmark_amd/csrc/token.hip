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

// a native 4-wide vector: arrays of it stay in registers (HIP's float4 is a
// struct that can keep an array of it in scratch memory)
typedef float f4 __attribute__((ext_vector_type(4)));

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
        // Keys are taken by physical position (sinks, then ring slots 0 ..
        // W-1), which needs no bookkeeping to address: the softmax does not
        // depend on their order.  Once meta is in, slots outside the window
        // are masked and the new row's key stands in at its slot.
        const int g = blockIdx.x / nsplit, sp = blockIdx.x % nsplit;
        const int k0 = sp * TOK_KEYS;
        float* base = nearp + (int64_t)g * nsplit * H * tok_rec(dv);
        const int LDK = d + 4, LDV = dv + 4;
        float* Kl = lds;                      // [64][d+4]
        float* Vl = Kl + TOK_KEYS * LDK;      // [64][dv+4]
        float* Ql = Vl + TOK_KEYS * LDV;      // [H][d]
        float* Pl = Ql + H * d;               // [H][64] scores, then weights
        float* ST = Pl + H * TOK_KEYS;        // [H][2] max, mass
        constexpr int NL = TOK_KEYS * (128 / 4) / TOK_THREADS;   // f4 per thread at d = 128
        constexpr int NQ = 16 * (128 / 4) / TOK_THREADS;         // queries, f4 per thread
        const f4 z4 = {0.f, 0.f, 0.f, 0.f};
        f4 kx[NL], vx[NL], qx[NQ];
        // every load is issued before the first use of any of them; the loads
        // take clamped (in-bounds) addresses and carry no condition, so no
        // load waits for another
        const int nkv = p.ns + p.W;
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int e = min(tid + u * TOK_THREADS, TOK_KEYS * (d / 4) - 1);
            const int row = e / (d / 4), c4 = (e % (d / 4)) * 4;
            const int x = min(k0 + row, nkv - 1);
            // both candidates computed, then selected: no branch around the loads
            const int xs = max(min(x, p.ns - 1), 0), xr = max(x - p.ns, 0);
            const float* ks = p.sink_k + ((int64_t)g * p.ns + xs) * d;
            const float* vs = p.sink_v + ((int64_t)g * p.ns + xs) * dv;
            const float* kr = p.ring_k + ((int64_t)g * p.W + xr) * d;
            const float* vr = p.ring_v + ((int64_t)g * p.W + xr) * dv;
            const float* kp = x < p.ns ? ks : kr;
            const float* vp = x < p.ns ? vs : vr;
            kx[u] = *reinterpret_cast<const f4*>(kp + c4);
            vx[u] = *reinterpret_cast<const f4*>(vp + c4);
        }
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            const int e = min(tid + u * TOK_THREADS, H * (d / 4) - 1);
            qx[u] = *reinterpret_cast<const f4*>(p.q + (int64_t)g * H * d + e * 4);
        }
        const bool nrow = tid < d / 4;   // threads that carry the new row's key and value
        const int tn = min(tid, d / 4 - 1);
        const f4 knew = *reinterpret_cast<const f4*>(p.k + (int64_t)g * d + tn * 4);
        const f4 vnew = *reinterpret_cast<const f4*>(p.v + (int64_t)g * dv + tn * 4);
        const GMeta c = load_gmeta(p.meta, g, p.W);
        const TokRow r = tok_row(c);
        // key x of this block is live: a sink, or a slot inside the window
        // after the push (written with no short-circuit and no division, so
        // that it compiles to selects rather than branches)
        auto live = [&](int x) {
            const int sl = x - p.ns;
            const int md = sl >= c.head0 ? sl - c.head0 : sl - c.head0 + c.wg;   // age order of slot sl
            return (x < nkv) & ((x < p.ns) | ((sl < c.wg) & (md < r.len1)));
        };
        const int xnew = p.ns + r.slot;   // where the new row's key sits
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int e = tid + u * TOK_THREADS;
            const int row = e / (d / 4), c4 = (e % (d / 4)) * 4;
            const int x = k0 + row;
            if (e < TOK_KEYS * (d / 4) && x != xnew) {   // the new row's threads write that row
                const bool ok = live(x);
                *reinterpret_cast<f4*>(Kl + row * LDK + c4) = ok ? kx[u] : z4;
                *reinterpret_cast<f4*>(Vl + row * LDV + c4) = ok ? vx[u] : z4;
            }
        }
        if (nrow && xnew >= k0 && xnew < k0 + TOK_KEYS) {
            *reinterpret_cast<f4*>(Kl + (xnew - k0) * LDK + tid * 4) = knew;
            *reinterpret_cast<f4*>(Vl + (xnew - k0) * LDV + tid * 4) = vnew;
        }
        const float qs = p.scale * TOK_LOG2E;
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            const int e = tid + u * TOK_THREADS;
            if (e < H * (d / 4))
                *reinterpret_cast<f4*>(Ql + e * 4) =
                    qx[u] * qs;
        }
        __syncthreads();
        // scores: thread per (head, key); dead keys score -inf
        for (int e = tid; e < H * TOK_KEYS; e += TOK_THREADS) {
            const int h = e / TOK_KEYS, j = e % TOK_KEYS;
            const int x = k0 + j;
            float acc = -INFINITY;
            if (live(x)) {
                const float* kr = Kl + j * LDK;
                const float* qr = Ql + h * d;
                acc = 0.f;
#pragma unroll 8
                for (int t = 0; t < d; t += 4) {
                    const f4 a = *reinterpret_cast<const f4*>(kr + t);
                    const f4 b = *reinterpret_cast<const f4*>(qr + t);
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
            const float pv = sc == -INFINITY ? 0.f : exp2f(sc - mx);
            const float l = wsum(pv);
            Pl[h * TOK_KEYS + lane] = pv;
            if (lane == 0) {
                ST[2 * h] = mx;
                ST[2 * h + 1] = l;
            }
        }
        __syncthreads();
        // value sums: thread per (head, value column); dead keys hold zero rows
        for (int e = tid; e < H * dv; e += TOK_THREADS) {
            const int h = e / dv, t = e % dv;
            const float* pr = Pl + h * TOK_KEYS;
            float acc = 0.f;
#pragma unroll 8
            for (int j = 0; j < TOK_KEYS; ++j) acc += pr[j] * Vl[j * LDV + t];
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
    float* KT = VE + dv;              // [64][d+4] landmark keys
    float* QT = KT + 64 * LDT;        // [16][d+4] this range's landmark queries
    float* TH = QT + TOK_BMAX * LDT;  // [16][dv]  this range's accumulators
    float* MU = TH + TOK_BMAX * dv;   // [64][16]  mu[a][b0 + j]
    float* EA = MU + 64 * TOK_BMAX;   // [64]      f_a, then e_a
    float* MB = EA + 64;              // [16]      M'
    float* RB = MB + 16;              // [16]      R
    float* XB = RB + 16;              // [16]      exp(l - M')
    float* ZB = XB + 16;              // [16]      Z'
    float* GB = ZB + 16;              // [16]      gains
    float* RED = GB + 16;             // [4]
    float* mz = p.mz + (int64_t)gh * 2 * m;
    const float* ring_k_e = p.ring_k + ((int64_t)g * p.W + c.head0) * d;
    const float* ring_v_e = p.ring_v + ((int64_t)g * p.W + c.head0) * dv;
    // every global load of the block is issued before the first LDS store
    constexpr int NKT = 64 * (128 / 4) / TOK_THREADS;         // landmark keys, f4 per thread
    constexpr int NQT = TOK_BMAX * (128 / 4) / TOK_THREADS;   // landmark queries
    constexpr int NTH = TOK_BMAX * (128 / 4) / TOK_THREADS;   // accumulators
    constexpr int NMU = 64 * TOK_BMAX / TOK_THREADS;          // mu entries
    const f4 z4 = {0.f, 0.f, 0.f, 0.f};
    f4 kt[NKT], qt[NQT], tv[NTH];
    float mu[NMU];
    // unconditional loads from clamped addresses (see the near blocks)
    const float qv = p.q[(int64_t)gh * d + min(tid, d - 1)];
    const float ke = ring_k_e[min(tid, d - 1)];
    const float ve = ring_v_e[min(tid, dv - 1)];
    const float* th_g = p.theta + ((int64_t)gh * m + b0) * dv;
#pragma unroll
    for (int u = 0; u < NKT; ++u) {
        const int e = tid + u * TOK_THREADS;
        const int a = min(e / (d / 4), m - 1), c4 = (e % (d / 4)) * 4;
        kt[u] = *reinterpret_cast<const f4*>(p.k_tilde + ((int64_t)g * m + a) * d + c4);
    }
#pragma unroll
    for (int u = 0; u < NQT; ++u) {
        const int e = tid + u * TOK_THREADS;
        const int j = min(e / (d / 4), nb - 1), c4 = (e % (d / 4)) * 4;
        qt[u] = *reinterpret_cast<const f4*>(p.q_tilde + ((int64_t)gh * m + b0 + j) * d + c4);
    }
#pragma unroll
    for (int u = 0; u < NTH; ++u) {
        const int e = min(tid + u * TOK_THREADS, nb * (dv / 4) - 1);
        tv[u] = *reinterpret_cast<const f4*>(th_g + e * 4);
    }
#pragma unroll
    for (int u = 0; u < NMU; ++u) {
        const int e = tid + u * TOK_THREADS;
        const int a = min(e / TOK_BMAX, m - 1), j = min(e % TOK_BMAX, nb - 1);
        mu[u] = p.mu[((int64_t)gh * m + a) * m + b0 + j];
    }
    if (tid < d) {
        Ql[tid] = qv;
        KE[tid] = r.full ? ke : 0.f;
    }
    if (tid < dv) VE[tid] = r.full ? ve : 0.f;
#pragma unroll
    for (int u = 0; u < NKT; ++u) {
        const int e = tid + u * TOK_THREADS;
        const int a = e / (d / 4), c4 = (e % (d / 4)) * 4;
        if (a < 64) *reinterpret_cast<f4*>(KT + a * LDT + c4) = a < m ? kt[u] : z4;
    }
#pragma unroll
    for (int u = 0; u < NQT; ++u) {
        const int e = tid + u * TOK_THREADS;
        const int j = e / (d / 4), c4 = (e % (d / 4)) * 4;
        if (j < TOK_BMAX) *reinterpret_cast<f4*>(QT + j * LDT + c4) = j < nb ? qt[u] : z4;
    }
#pragma unroll
    for (int u = 0; u < NTH; ++u) {
        const int e = tid + u * TOK_THREADS;
        if (e < TOK_BMAX * (dv / 4)) *reinterpret_cast<f4*>(TH + e * 4) = e < nb * (dv / 4) ? tv[u] : z4;
    }
#pragma unroll
    for (int u = 0; u < NMU; ++u) {
        const int e = tid + u * TOK_THREADS;
        MU[e] = (e / TOK_BMAX < m && e % TOK_BMAX < nb) ? mu[u] : 0.f;
    }
    __syncthreads();
    // f_a (base 2) for every landmark: 4 lanes per landmark
    for (int e = tid; e < 64 * 4; e += TOK_THREADS) {
        const int a = e >> 2, qq = e & 3;
        float acc = 0.f;
        if (a < m) {
            const float* kr = KT + a * LDT;
            for (int t = qq * 4; t < d; t += 16) {
                const f4 x = *reinterpret_cast<const f4*>(kr + t);
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
                const f4 y = *reinterpret_cast<const f4*>(qr + t);
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
// part dropped when its total mass is not >= 0, out.  Thread (column, part)
// folds records part, part + P, ... of the head with a running exponent (all
// of its loads for up to TOK_MB records issued at once); the parts then meet
// in LDS.  The first head of a group also pushes the row into the ring and
// advances meta (no other block of this kernel reads them).
constexpr int TOK_MT = 512;   // merge threads
constexpr int TOK_MB = 16;    // records per thread per batch of loads

__global__ __launch_bounds__(TOK_MT) void k_tok_merge(KParams p, const float* part, int nsplit)
{
    extern __shared__ float lds[];
    const int gh = blockIdx.x, g = gh / p.H, h = gh % p.H;
    const int tid = threadIdx.x;
    const int H = p.H, dv = p.dv;
    const int64_t rl = tok_rec(dv);
    const float* nearp = part + (int64_t)g * nsplit * H * rl + (int64_t)h * rl;   // stride H*rl
    const float* farp = part + (int64_t)p.G * nsplit * H * rl + (int64_t)gh * TOK_FB * rl;
    const int P = TOK_MT / dv;                   // dv divides TOK_MT
    const int col = tid % dv, prt = tid / dv;
    float* SM = lds;                             // [P+1] exponent of each part; the far part last
    float* SL = SM + P + 1;                      // [P+1] mass
    float* SA = SL + P + 1;                      // [P+1][dv] value sums
    // the far ranges: every thread reads them (their loads go out with the
    // near records').  Their total mass is taken against their own largest
    // exponent: its sign does not depend on the exponent.
    float fmk[TOK_FB], flk[TOK_FB], fxk[TOK_FB];
#pragma unroll
    for (int j = 0; j < TOK_FB; ++j) {
        fmk[j] = farp[j * rl];
        flk[j] = farp[j * rl + 1];
        fxk[j] = farp[j * rl + 2 + col];
    }
    float mrun = -INFINITY, lrun = 0.f, acc = 0.f;
    // records k0, k0 + P, ..., k0 + (TOK_MB-1) P, folded in with a running exponent
    auto fold = [&](int k0) {
        float ms[TOK_MB], ls[TOK_MB], xs[TOK_MB];
#pragma unroll
        for (int u = 0; u < TOK_MB; ++u) {
            const int k = k0 + u * P;
            const float* rc = nearp + (int64_t)min(k, nsplit - 1) * H * rl;   // clamped: no condition on the loads
            ms[u] = rc[0];
            ls[u] = rc[1];
            xs[u] = rc[2 + col];
        }
#pragma unroll
        for (int u = 0; u < TOK_MB; ++u)
            if (k0 + u * P >= nsplit) ms[u] = -INFINITY;
        float bm = mrun;
#pragma unroll
        for (int u = 0; u < TOK_MB; ++u) bm = fmaxf(bm, ms[u]);
        // no early exit when every record is empty: the loads stay unconditional
        const float bx = bm == -INFINITY ? 0.f : bm;
        const float sc = mrun == -INFINITY ? 0.f : exp2f(mrun - bx);
        acc *= sc;
        lrun *= sc;
#pragma unroll
        for (int u = 0; u < TOK_MB; ++u) {
            const float w = ms[u] == -INFINITY ? 0.f : exp2f(ms[u] - bx);
            acc += w * xs[u];
            lrun += w * ls[u];
        }
        mrun = bm;
    };
    fold(prt);   // the first batch in straight-line code, so its loads go out with the far ones
    for (int k0 = prt + TOK_MB * P; k0 < nsplit; k0 += TOK_MB * P) fold(k0);
    SA[prt * dv + col] = acc;
    if (col == 0) {
        SM[prt] = mrun;
        SL[prt] = lrun;
    }
    if (prt == 0) {
        float fm = -INFINITY;
#pragma unroll
        for (int j = 0; j < TOK_FB; ++j) fm = fmaxf(fm, fmk[j]);
        float dfar = 0.f, xfar = 0.f;
#pragma unroll
        for (int j = 0; j < TOK_FB; ++j) {
            const float w = fmk[j] == -INFINITY ? 0.f : exp2f(fmk[j] - fm);
            dfar += w * flk[j];
            xfar += w * fxk[j];
        }
        const bool have = fm != -INFINITY && dfar >= 0.f;   // else the far part is dropped
        SA[P * dv + col] = have ? xfar : 0.f;
        if (col == 0) {
            SM[P] = have ? fm : -INFINITY;
            SL[P] = have ? dfar : 0.f;
        }
    }
    __syncthreads();
    if (tid < dv) {
        float c = -INFINITY;
        for (int q = 0; q <= P; ++q) c = fmaxf(c, SM[q]);
        float den = 0.f, num = 0.f;
        for (int q = 0; q <= P; ++q) {
            const float w = SM[q] == -INFINITY ? 0.f : exp2f(SM[q] - c);
            den += w * SL[q];
            num += w * SA[q * dv + tid];
        }
        p.out[(int64_t)gh * dv + tid] = num / fmaxf(den, 1e-30f);
    }
    if (h == 0) {
        // commit: ring push and meta (every reader of the ring and meta of
        // this group ran in the previous kernel)
        const GMeta c = load_gmeta(p.meta, g, p.W);
        const TokRow r = tok_row(c);
        __syncthreads();   // all threads have read meta before thread 0 writes it
        float* kd = p.ring_k + ((int64_t)g * p.W + r.slot) * p.d;
        float* vd = p.ring_v + ((int64_t)g * p.W + r.slot) * dv;
        for (int e = tid; e < p.d; e += TOK_MT) kd[e] = p.k[(int64_t)g * p.d + e];
        for (int e = tid; e < dv; e += TOK_MT) vd[e] = p.v[(int64_t)g * dv + e];
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
    const size_t lds_far = sizeof(float) * ((size_t)2 * p.d + p.dv + (size_t)64 * (p.d + 4) +
                                            (size_t)TOK_BMAX * (p.d + 4) + (size_t)TOK_BMAX * p.dv +
                                            (size_t)64 * TOK_BMAX + 64 + 5 * 16 + 4);
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
    const size_t lds_merge = sizeof(float) * ((size_t)(TOK_MT / p.dv + 1) * (p.dv + 2));
    hipLaunchKernelGGL(k_tok_merge, dim3(p.nh), dim3(TOK_MT), lds_merge, st, p,
                       (const float*)part, nsplit);
    return hipGetLastError();
}

}  // namespace swl
