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
#include "lanes.h"

namespace swl {

constexpr int TOK_KEYS = 64;    // keys per near block
constexpr int TOK_FB = 4;       // far blocks per query head (landmark ranges)
constexpr int TOK_BMAX = 16;    // landmarks per far block (m <= 64)
constexpr int TOK_THREADS = 512;
constexpr float TOK_LOG2E = 1.4426950408889634f;

// a native 4-wide vector: arrays of it stay in registers (HIP's float4 is a
// struct that can keep an array of it in scratch memory)
typedef float f4 __attribute__((ext_vector_type(4)));

int tok_splits(int ns, int W) { return (ns + W + TOK_KEYS - 1) / TOK_KEYS; }

// partial record: [0] max (base 2), [1] mass, [4 .. 4+dv) value sum (16-byte aligned)
constexpr int TOK_V0 = 4;
__host__ __device__ inline int64_t tok_rec(int dv) { return TOK_V0 + dv; }

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

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// Sum, over groups of L lanes (L a power of two; the lanes of a group differ
// only in their low log2 L bits), of N partial values held by each lane.
// While a lane holds more than one value, each step hands half of them to the
// partner lane and keeps the other half (a reduce-scatter); once one is left,
// the remaining steps add it across.  Afterwards slot i (i < slots) of lane
// li holds the group sum of original index index(i, li).  The steps are
// template recursions, so that every array index is a constant from the
// start (a select between two elements must not become a per-lane index).
template <int N, int L>
struct LaneReduce {
    static constexpr int slots = N >= L ? N / L : 1;
    static constexpr int share = L > N ? L / N : 1;   // lanes holding the same sum
    __device__ static int index(int i, int li) { return i + (li / share) * slots; }

    template <int I, int HALF, int B>
    __device__ static void pairs(float (&v)[N], int lane)
    {
        if constexpr (I < HALF) {
            v[I] = pair_split<B>(v[I], v[I + HALF], lane);
            pairs<I + 1, HALF, B>(v, lane);
        }
    }
    template <int B, int n>   // bit of the partner lane, values held
    __device__ static void step(float (&v)[N], int lane)
    {
        if constexpr (B >= 0) {
            if constexpr (n > 1)
                pairs<0, n / 2, B>(v, lane);
            else
                v[0] = pair_sum<B>(v[0]);
            step<B - 1, (n > 1 ? n / 2 : 1)>(v, lane);
        }
    }
    // lane: the lane index in the wave (its low log2 L bits are the index in the group)
    __device__ static void run(float (&v)[N], int lane) { step<ilog2(L) - 1, N>(v, lane); }
};

// Sum of each value over the lanes of a wave that differ in bits B .. 5 (the
// row groups of the wave), lanes below bit B kept apart.
template <int B, int HC>
__device__ __forceinline__ void rows_sum(f4 (&acc)[HC])
{
    if constexpr (B <= 5) {
#pragma unroll
        for (int j = 0; j < HC; ++j) {
            acc[j].x = xor_sum<B>(acc[j].x);
            acc[j].y = xor_sum<B>(acc[j].y);
            acc[j].z = xor_sum<B>(acc[j].z);
            acc[j].w = xor_sum<B>(acc[j].w);
        }
        rows_sum<B + 1>(acc);
    }
}

// 2^x by the hardware instruction: arguments here are <= 0 (against a
// maximum), and results below 2^-126 may flush to zero
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float dot4(f4 a, f4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }

// Elements c4 .. c4+3 of the row's query or key head x, turned by the RoPE
// table row tab when there is one.
__device__ __forceinline__ f4 tok_in(const float* x, const float* tab, int c4, int D)
{
    const float4 v = rope4(x, tab, c4, D);
    return f4{v.x, v.y, v.z, v.w};
}

// Near partial of group g, keys k0 .. k0+63 taken by physical position (the
// sinks, then ring slots 0 .. W-1), which needs no bookkeeping to address:
// the softmax does not depend on their order.  Thread (rb, li) holds columns
// 4li .. 4li+3 of key rows rb, rb + RPP, ... in registers, straight from
// global memory: scores are lane-group sums, and the value sums are formed in
// registers and summed over the block through LDS.  Once meta is in, slots
// outside the window are masked and the new row's key stands in at its slot.
template <int D>
__device__ __forceinline__ void tok_near(const KParams& p, float* nearp, int nsplit, int blk, float* lds)
{
    constexpr int L = D / 4;                                   // lanes per key row
    constexpr int RPP = TOK_THREADS / L;                       // key rows per pass
    constexpr int NL = RPP >= TOK_KEYS ? 1 : TOK_KEYS / RPP;   // passes
    constexpr int HC = 4;                                      // heads per chunk
    using LR = LaneReduce<NL * HC, L>;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = tid % L, rb = tid / L, c4 = li * 4;
    const int H = p.H;
    const int g = blk / nsplit, sp = blk % nsplit, k0 = sp * TOK_KEYS;
    const int nkv = p.ns + p.W;
    float* SC = lds;                  // [H][64] scores, then weights
    float* ST = SC + H * TOK_KEYS;    // [16][2] max, mass
    float* PS = ST + 32;              // [waves][4][D] value sums of each wave, for a chunk of 4 heads
    const f4 z4 = {0.f, 0.f, 0.f, 0.f};
    // every load is issued before the first use of any of them: clamped
    // (in-bounds) addresses, no condition on the loads
    f4 kx[NL], vx[NL], q0[HC];
#pragma unroll
    for (int u = 0; u < NL; ++u) {
        const int row = min(rb + u * RPP, TOK_KEYS - 1);
        const int x = min(k0 + row, nkv - 1);
        // both candidates computed, then selected: no branch around the loads
        const int xs = max(min(x, p.ns - 1), 0), xr = max(x - p.ns, 0);
        const float* ks = p.sink_k + ((int64_t)g * p.ns + xs) * D;
        const float* vs = p.sink_v + ((int64_t)g * p.ns + xs) * D;
        const float* kr = p.ring_k + ((int64_t)g * p.W + xr) * D;
        const float* vr = p.ring_v + ((int64_t)g * p.W + xr) * D;
        kx[u] = *reinterpret_cast<const f4*>((x < p.ns ? ks : kr) + c4);
        vx[u] = *reinterpret_cast<const f4*>((x < p.ns ? vs : vr) + c4);
    }
#pragma unroll
    for (int j = 0; j < HC; ++j) q0[j] = tok_in(p.q + ((int64_t)g * H + min(j, H - 1)) * D, p.rope, c4, D);
    const f4 knew = tok_in(p.k + (int64_t)g * D, p.rope, c4, D);
    const f4 vnew = *reinterpret_cast<const f4*>(p.v + (int64_t)g * D + c4);
    const GMeta c = load_gmeta(p.meta, g, p.W);
    const TokRow r = tok_row(c);
    // key x is live: a sink, or a slot inside the window after the push
    // (no short-circuit and no division: selects rather than branches)
    auto live = [&](int x) {
        const int sl = x - p.ns;
        const int md = sl >= c.head0 ? sl - c.head0 : sl - c.head0 + c.wg;   // age order of slot sl
        return (x < nkv) & ((x < p.ns) | ((sl < c.wg) & (md < r.len1)));
    };
    const int xnew = p.ns + r.slot;   // where the new row's key sits
#pragma unroll
    for (int u = 0; u < NL; ++u) {
        const int row = rb + u * RPP, x = k0 + row;
        const bool ok = (row < TOK_KEYS) & live(x), nw = (row < TOK_KEYS) & (x == xnew);
        kx[u] = nw ? knew : (ok ? kx[u] : z4);   // dead rows hold zeros (their memory may hold anything)
        vx[u] = nw ? vnew : (ok ? vx[u] : z4);
    }
    const float qs = p.scale * TOK_LOG2E;   // scores in base 2
    for (int hc = 0; hc < H; hc += HC) {
        f4 qc[HC];
#pragma unroll
        for (int j = 0; j < HC; ++j)
            qc[j] = hc == 0 ? q0[j] : tok_in(p.q + ((int64_t)g * H + min(hc + j, H - 1)) * D, p.rope, c4, D);
        float s[NL * HC];
#pragma unroll
        for (int u = 0; u < NL; ++u)
#pragma unroll
            for (int j = 0; j < HC; ++j) s[u * HC + j] = dot4(kx[u], qc[j]);
        LR::run(s, lane);
#pragma unroll
        for (int i = 0; i < LR::slots; ++i) {
            const int idx = LR::index(i, li), u = idx / HC, h = hc + idx % HC, row = rb + u * RPP;
            if (li % LR::share == 0 && row < TOK_KEYS && h < H)
                SC[h * TOK_KEYS + row] = live(k0 + row) ? s[i] * qs : -INFINITY;
        }
    }
    __syncthreads();
    // per head: max, weights, mass (a wave per head, lane = key)
    for (int h = wave; h < H; h += TOK_THREADS / 64) {
        const float sc = lane < TOK_KEYS ? SC[h * TOK_KEYS + lane] : -INFINITY;
        const float mx = wmax(sc);
        const float pv = sc == -INFINITY ? 0.f : ex2(sc - mx);
        const float l = wsum(pv);
        if (lane < TOK_KEYS) SC[h * TOK_KEYS + lane] = pv;
        if (lane == 0) {
            ST[2 * h] = mx;
            ST[2 * h + 1] = l;
        }
    }
    __syncthreads();
    // value sums: registers, then over the row groups of the wave, then over
    // the waves through LDS, a chunk of HC heads at a time
    constexpr int NWV = TOK_THREADS / 64;
    float* base = nearp + (int64_t)g * nsplit * H * tok_rec(D);
    for (int hc = 0; hc < H; hc += HC) {
        f4 acc[HC];
#pragma unroll
        for (int j = 0; j < HC; ++j) acc[j] = z4;
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int row = min(rb + u * RPP, TOK_KEYS - 1);   // rows past the block hold zero values
#pragma unroll
            for (int j = 0; j < HC; ++j)   // heads past H repeat the last one; their sums are dropped
                acc[j] += SC[min(hc + j, H - 1) * TOK_KEYS + row] * vx[u];
        }
        rows_sum<ilog2(L)>(acc);
        if (hc > 0) __syncthreads();   // the previous chunk's sums have been read
        if (lane < L)
#pragma unroll
            for (int j = 0; j < HC; ++j) *reinterpret_cast<f4*>(PS + ((int64_t)wave * HC + j) * D + c4) = acc[j];
        __syncthreads();
        for (int e = tid; e < HC * (D / 4); e += TOK_THREADS) {
            const int j = e / (D / 4), t = (e % (D / 4)) * 4, h = hc + j;
            if (h < H) {
                f4 a = *reinterpret_cast<const f4*>(PS + (int64_t)j * D + t);
#pragma unroll
                for (int w = 1; w < NWV; ++w) a += *reinterpret_cast<const f4*>(PS + ((int64_t)w * HC + j) * D + t);
                float* rec = base + ((int64_t)sp * H + h) * tok_rec(D);
                *reinterpret_cast<f4*>(rec + TOK_V0 + t) = a;
                if (t == 0) {
                    rec[0] = ST[2 * h];
                    rec[1] = ST[2 * h + 1];
                }
            }
        }
    }
}

// Far partial of query head gh over landmark range fb.  When the ring is full
// the row evicts the key at slot head; every landmark b of the range folds it
// in (l = scale <q~_b, k_e>, M' = max(M, l), R = 1 if M' == M else e^{M-M'},
// Z' = R Z + e^{l-M'}, Theta' = R Theta + e^{l-M'} v_e) and writes M', Z',
// Theta' back.  Then the far estimate of the range against M': u_b = sum_a
// e^{f_a-f_max} mu[a][b] (>= 0 with rect), gain_b against the range's own
// exponent, D = sum_b gain_b Z'_b and N = sum_b gain_b Theta'_b -- for a
// one-row chunk the chunk form's R Theta + cf v_e is exactly Theta'.  The
// landmark keys and queries stay in registers (lane-group sums, as in the
// near blocks); the accumulators and mu pass through LDS.
template <int D>
__device__ __forceinline__ void tok_far(const KParams& p, float* farp, int fbk, float* lds)
{
    constexpr int L = D / 4, RPP = TOK_THREADS / L;
    constexpr int NK = RPP >= 64 ? 1 : 64 / RPP;                 // landmark-key passes (m <= 64)
    constexpr int NQ = RPP >= TOK_BMAX ? 1 : TOK_BMAX / RPP;     // landmark-query passes
    constexpr int NTH = (TOK_BMAX * (D / 4) + TOK_THREADS - 1) / TOK_THREADS;   // accumulator pieces per thread
    constexpr int NMU = 64 * TOK_BMAX / TOK_THREADS;
    using LRK = LaneReduce<NK, L>;
    using LRQ = LaneReduce<NQ, L>;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int li = tid % L, rb = tid / L, c4 = li * 4;
    const int H = p.H, m = p.m;
    const int gh = fbk / TOK_FB, fb = fbk % TOK_FB, g = gh / H;
    const GMeta c = load_gmeta(p.meta, g, p.W);
    const TokRow r = tok_row(c);
    float* rec = farp + ((int64_t)gh * TOK_FB + fb) * tok_rec(D);
    const int per = (m + TOK_FB - 1) / TOK_FB;   // <= TOK_BMAX
    const int b0 = fb * per, b1 = min(m, b0 + per), nb = b1 - b0;
    if (r.nfar1 == 0 || nb <= 0) {
        for (int t = tid; t < tok_rec(D); t += TOK_THREADS) rec[t] = t == 0 ? -INFINITY : 0.f;
        return;
    }
    constexpr int C4 = D / 4;
    static_assert(TOK_THREADS % C4 == 0, "a thread's accumulator pieces share one column");
    float* MU = lds;                  // [64][16]  mu[a][b0 + j]
    float* VE = MU + 64 * TOK_BMAX;   // [D]       evicted value
    float* NS = VE + D;               // [waves][D] value sums of each wave
    float* EA = NS + (TOK_THREADS / 64) * D;   // [64] f_a, then e_a (0 past m)
    float* LB = EA + 64;              // [16]      evicted key's score per landmark
    float* MB = LB + 16;              // [16]      M'
    float* RB = MB + 16;              // [16]      R
    float* XB = RB + 16;              // [16]      exp(l - M')
    float* ZB = XB + 16;              // [16]      Z'
    float* GB = ZB + 16;              // [16]      gains
    float* RED = GB + 16;             // [4]
    float* mz = p.mz + (int64_t)gh * 2 * m;
    const f4 z4 = {0.f, 0.f, 0.f, 0.f};
    // loads, unconditional from clamped addresses; the evicted key's come
    // last, as their address needs meta
    f4 kt[NK], qt[NQ], tv[NTH];
    float mu[NMU];
#pragma unroll
    for (int u = 0; u < NK; ++u) {
        const int a = min(rb + u * RPP, m - 1);
        kt[u] = *reinterpret_cast<const f4*>(p.k_tilde + ((int64_t)g * m + a) * D + c4);
    }
    const f4 qh = tok_in(p.q + (int64_t)gh * D, p.rope, c4, D);
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
        const int j = min(rb + u * RPP, nb - 1);
        qt[u] = *reinterpret_cast<const f4*>(p.q_tilde + ((int64_t)gh * m + b0 + j) * D + c4);
    }
    const float* th_g = p.theta + ((int64_t)gh * m + b0) * D;
#pragma unroll
    for (int u = 0; u < NTH; ++u) {
        const int e = min(tid + u * TOK_THREADS, nb * (D / 4) - 1);
        tv[u] = *reinterpret_cast<const f4*>(th_g + e * 4);
    }
#pragma unroll
    for (int u = 0; u < NMU; ++u) {
        const int e = tid + u * TOK_THREADS;
        const int a = min(e / TOK_BMAX, m - 1), j = min(e % TOK_BMAX, nb - 1);
        mu[u] = p.mu[((int64_t)gh * m + a) * m + b0 + j];
    }
    const int bj = b0 + min(tid, nb - 1);
    const float Mo = mz[bj], Zo = mz[m + bj];
    const f4 ke = *reinterpret_cast<const f4*>(p.ring_k + ((int64_t)g * p.W + c.head0) * D + c4);
    const float ve = p.ring_v[((int64_t)g * p.W + c.head0) * D + min(tid, D - 1)];
    // LDS: mu, evicted value (the accumulators stay in registers)
#pragma unroll
    for (int u = 0; u < NMU; ++u) {
        const int e = tid + u * TOK_THREADS;
        MU[e] = (e / TOK_BMAX < m && e % TOK_BMAX < nb) ? mu[u] : 0.f;
    }
    if (tid < D) VE[tid] = r.full ? ve : 0.f;
    // f_a (base 2) for every landmark, and the evicted key's score per landmark of the range
    {
        float s[NK];
#pragma unroll
        for (int u = 0; u < NK; ++u) s[u] = dot4(kt[u], qh);
        LRK::run(s, lane);
#pragma unroll
        for (int i = 0; i < LRK::slots; ++i) {
            const int a = rb + LRK::index(i, li) * RPP;
            if (li % LRK::share == 0 && a < m) EA[a] = s[i] * p.scale * TOK_LOG2E;
        }
        float t[NQ];
#pragma unroll
        for (int u = 0; u < NQ; ++u) t[u] = dot4(qt[u], ke);
        LRQ::run(t, lane);
#pragma unroll
        for (int i = 0; i < LRQ::slots; ++i) {
            const int j = rb + LRQ::index(i, li) * RPP;
            if (li % LRQ::share == 0 && j < nb) LB[j] = t[i] * p.scale;
        }
    }
    __syncthreads();
    // the fold, a thread per landmark of the range
    if (tid < nb) {
        float Mn = Mo, R = 1.f, x = 0.f, Zn = Zo;
        if (r.full) {
            const float l = LB[tid];
            Mn = fmaxf(Mo, l);
            R = (Mn == Mo) ? 1.f : expf(Mo - Mn);
            x = expf(l - Mn);
            Zn = Zo * R + x;
            mz[bj] = Mn;
            mz[m + bj] = Zn;
        }
        MB[tid] = Mn;
        RB[tid] = R;
        XB[tid] = x;
        ZB[tid] = Zn;
    }
    if (wave == 1) {
        const float f = lane < m ? EA[lane] : -INFINITY;
        const float fmax = wmax(f);
        EA[lane] = lane < m ? ex2(f - fmax) : 0.f;
        if (lane == 0) RED[0] = fmax;
    }
    __syncthreads();
    if (wave == 0) {
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
#pragma unroll
        for (int a = qq; a < 64; a += 16) u += EA[a] * MU[a * TOK_BMAX + min(j, TOK_BMAX - 1)];   // zeros past m
        u = sum16(u);
        if (qq == 0 && j < nb) {
            if (p.rect) u = fmaxf(u, 0.f);
            GB[j] = u * ex2(fmax + MB[j] * TOK_LOG2E - cl);
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
    // Theta' = R Theta + x v_e (written back) and N = sum_b gain_b Theta'_b:
    // thread (j, cc) holds columns 4cc .. 4cc+3 of accumulator b0 + j (two
    // such pieces at d = 256)
    {
        const int cc = tid % C4;   // the same column for every piece of this thread
        f4 y[1] = {z4};
#pragma unroll
        for (int u = 0; u < NTH; ++u) {
            const int e = tid + u * TOK_THREADS, j = e / C4;
            if (e < TOK_BMAX * C4 && j < nb) {
                f4 x = tv[u];
                if (r.full) {
                    x = x * RB[j] + XB[j] * *reinterpret_cast<const f4*>(VE + cc * 4);
                    *reinterpret_cast<f4*>(p.theta + ((int64_t)gh * m + b0 + j) * D + cc * 4) = x;
                }
                y[0] += GB[j] * x;
            }
        }
        rows_sum<ilog2(C4)>(y);   // over the accumulators of the wave
        if (lane < C4) *reinterpret_cast<f4*>(NS + (int64_t)wave * D + cc * 4) = y[0];
        __syncthreads();
        if (tid < C4) {
            f4 a = *reinterpret_cast<const f4*>(NS + tid * 4);
#pragma unroll
            for (int w = 1; w < TOK_THREADS / 64; ++w) a += *reinterpret_cast<const f4*>(NS + (int64_t)w * D + tid * 4);
            *reinterpret_cast<f4*>(rec + TOK_V0 + tid * 4) = a;
        }
    }
}

template <int D>
__global__ __launch_bounds__(TOK_THREADS) void k_tok_part(KParams p, float* part, int nsplit)
{
    extern __shared__ float lds[];
    const int nnear = p.G * nsplit;
    if ((int)blockIdx.x < nnear)
        tok_near<D>(p, part, nsplit, blockIdx.x, lds);
    else
        tok_far<D>(p, part + (int64_t)nnear * p.H * tok_rec(D), blockIdx.x - nnear, lds);
}

// One block per query head: the head's partials to one exponent c = max of
// all partial maxima (the pages' c = max(c_near, f_max + M'_b)), the far part
// dropped when its total mass is not >= 0, out = (N + sum p v) / max(D + sum
// p, 1e-30).  Thread (part, c4) folds records part, part + NPRT, ... with a
// running exponent, reading each record's head and columns 4c4 .. 4c4+3 as
// 16-byte loads; parts 0 .. 3 also take one far range each.  The parts meet
// in LDS.  The first head of a group then pushes the row into the ring (slot
// head when the ring is full, else head + len) and advances meta: no other
// block of this kernel reads them, and every reader ran in the previous one.
// Two partials (exponent m, mass l, value sums a) to one, against the larger
// exponent; either may be empty (m = -inf).
__device__ __forceinline__ void merge2(float& m, float& l, f4& a, float m2, float l2, f4 a2)
{
    const float mn = fmaxf(m, m2);
    const float w1 = m == -INFINITY ? 0.f : ex2(m - mn), w2 = m2 == -INFINITY ? 0.f : ex2(m2 - mn);
    l = l * w1 + l2 * w2;
    a = a * w1 + a2 * w2;
    m = mn;
}

// merge2 over the lanes of a wave that differ in bits B .. 5, lanes below bit
// B kept apart; every lane of such a set ends with the same result
template <int B>
__device__ __forceinline__ void wave_merge(float& m, float& l, f4& a, int lane)
{
    if constexpr (B <= 5) {
        f4 a2;
        a2.x = xor_get<B>(a.x, lane);
        a2.y = xor_get<B>(a.y, lane);
        a2.z = xor_get<B>(a.z, lane);
        a2.w = xor_get<B>(a.w, lane);
        merge2(m, l, a, xor_get<B>(m, lane), xor_get<B>(l, lane), a2);
        wave_merge<B + 1>(m, l, a, lane);
    }
}

constexpr int TOK_MT = 512;   // merge threads
constexpr int TOK_MB = 4;     // records per thread per batch of loads

template <int D>
__global__ __launch_bounds__(TOK_MT) void k_tok_merge(KParams p, const float* part, int nsplit)
{
    constexpr int C4 = D / 4;              // 16-byte columns
    constexpr int NPRT = TOK_MT / C4;      // parts (>= 16 > TOK_FB)
    extern __shared__ float lds[];
    const int gh = blockIdx.x, H = p.H, g = gh / H, h = gh % H;
    const int tid = threadIdx.x, c4 = tid % C4, prt = tid / C4;
    const int64_t rl = tok_rec(D);
    const float* nearp = part + ((int64_t)g * nsplit * H + h) * rl;   // record k at k * H * rl
    const float* farp = part + (int64_t)p.G * nsplit * H * rl + (int64_t)gh * TOK_FB * rl;
    constexpr int NW = TOK_MT / 64;        // waves
    float* SM = lds;                       // [NW + TOK_FB] exponent of each wave, then of each far range
    float* SL = SM + 16;                   // [NW + TOK_FB] mass
    float* SA = SL + 16;                   // [NW + TOK_FB][D] value sums
    // the commit's loads go out with the others (every block issues them;
    // only the first head of a group stores)
    const GMeta c = load_gmeta(p.meta, g, p.W);
    const f4 kn = tok_in(p.k + (int64_t)g * D, p.rope, c4 * 4, D);
    const f4 vn = *reinterpret_cast<const f4*>(p.v + (int64_t)g * D + c4 * 4);
    // far range prt (parts 0 .. TOK_FB-1), loaded unconditionally
    const float* fr = farp + (int64_t)min(prt, TOK_FB - 1) * rl;
    const f4 fh = *reinterpret_cast<const f4*>(fr);
    const f4 fx = *reinterpret_cast<const f4*>(fr + TOK_V0 + c4 * 4);
    const f4 z4 = {0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.f;
    f4 acc = z4;
    // records k0, k0 + NPRT, ..., folded in with a running exponent
    auto fold = [&](int k0) {
        f4 hd[TOK_MB], xs[TOK_MB];
#pragma unroll
        for (int u = 0; u < TOK_MB; ++u) {
            const float* rc = nearp + (int64_t)min(k0 + u * NPRT, nsplit - 1) * H * rl;   // clamped: no condition
            hd[u] = *reinterpret_cast<const f4*>(rc);
            xs[u] = *reinterpret_cast<const f4*>(rc + TOK_V0 + c4 * 4);
        }
        float ms[TOK_MB];
        float bm = mrun;
#pragma unroll
        for (int u = 0; u < TOK_MB; ++u) {
            ms[u] = k0 + u * NPRT < nsplit ? hd[u].x : -INFINITY;
            bm = fmaxf(bm, ms[u]);
        }
        // no early exit when every record is empty: the loads stay unconditional
        const float bx = bm == -INFINITY ? 0.f : bm;
        const float sc = mrun == -INFINITY ? 0.f : ex2(mrun - bx);
        acc *= sc;
        lrun *= sc;
#pragma unroll
        for (int u = 0; u < TOK_MB; ++u) {
            const float w = ms[u] == -INFINITY ? 0.f : ex2(ms[u] - bx);
            acc += w * xs[u];
            lrun += w * hd[u].y;
        }
        mrun = bm;
    };
    fold(prt);   // the first batch in straight-line code, so its loads go out with the rest
    for (int k0 = prt + TOK_MB * NPRT; k0 < nsplit; k0 += TOK_MB * NPRT) fold(k0);
    // the parts of a wave meet by lane exchanges (lanes that differ in the
    // bits above the column bits), then the waves and the far ranges in LDS
    wave_merge<ilog2(C4)>(mrun, lrun, acc, tid & 63);
    const int wave = tid >> 6;
    if ((tid & 63) < C4) {
        *reinterpret_cast<f4*>(SA + (int64_t)wave * D + c4 * 4) = acc;
        if (c4 == 0) {
            SM[wave] = mrun;
            SL[wave] = lrun;
        }
    }
    if (prt < TOK_FB) {
        *reinterpret_cast<f4*>(SA + (int64_t)(NW + prt) * D + c4 * 4) = fx;
        if (c4 == 0) {
            SM[NW + prt] = fh.x;
            SL[NW + prt] = fh.y;
        }
    }
    __syncthreads();
    if (tid < C4) {
        float sm[NW + TOK_FB], sl[NW + TOK_FB];
        f4 sa[NW + TOK_FB];
#pragma unroll
        for (int q = 0; q < NW + TOK_FB; ++q) {
            sm[q] = SM[q];
            sl[q] = SL[q];
            sa[q] = *reinterpret_cast<const f4*>(SA + (int64_t)q * D + tid * 4);
        }
        // the far ranges' total mass against their own largest exponent: its
        // sign does not depend on the exponent
        float fm = -INFINITY;
#pragma unroll
        for (int j = NW; j < NW + TOK_FB; ++j) fm = fmaxf(fm, sm[j]);
        float dfar = 0.f;
#pragma unroll
        for (int j = NW; j < NW + TOK_FB; ++j)
            dfar += sm[j] == -INFINITY ? 0.f : sl[j] * ex2(sm[j] - fm);
        const bool have = fm != -INFINITY && dfar >= 0.f;   // else the far part is dropped
#pragma unroll
        for (int j = NW; j < NW + TOK_FB; ++j)
            if (!have) sm[j] = -INFINITY;
        float cm = -INFINITY;
#pragma unroll
        for (int q = 0; q < NW + TOK_FB; ++q) cm = fmaxf(cm, sm[q]);
        float den = 0.f;
        f4 num = z4;
#pragma unroll
        for (int q = 0; q < NW + TOK_FB; ++q) {
            const float w = sm[q] == -INFINITY ? 0.f : ex2(sm[q] - cm);
            den += w * sl[q];
            num += w * sa[q];
        }
        f4 o = num * (1.f / fmaxf(den, 1e-30f));
        if (p.gate) {   // the output gate, when on
            const f4 z = *reinterpret_cast<const f4*>(p.gate + (int64_t)gh * D + tid * 4);
            const f4 s = *reinterpret_cast<const f4*>(p.gate_scale + (int64_t)gh * D + tid * 4);
            o = f4{o.x * gate_of(z.x, s.x), o.y * gate_of(z.y, s.y), o.z * gate_of(z.z, s.z), o.w * gate_of(z.w, s.w)};
        }
        *reinterpret_cast<f4*>(p.out + (int64_t)gh * D + tid * 4) = o;
        if (h == 0) {
            const TokRow r = tok_row(c);
            *reinterpret_cast<f4*>(p.ring_k + ((int64_t)g * p.W + r.slot) * D + tid * 4) = kn;
            *reinterpret_cast<f4*>(p.ring_v + ((int64_t)g * p.W + r.slot) * D + tid * 4) = vn;
            if (tid == 0) {
                p.meta[4 * g + 0] = (uint32_t)r.len1;
                p.meta[4 * g + 1] = (uint32_t)r.head1;
                p.meta[4 * g + 2] = (uint32_t)r.nfar1;
            }
        }
    }
}

// the partial kernel, then the merge
template <int D>
static hipError_t launch_two(const KParams& p, float* part, int nsplit, hipStream_t st)
{
    const size_t lds_near = sizeof(float) * ((size_t)p.H * TOK_KEYS + 32 + (size_t)(TOK_THREADS / 64) * 4 * D);
    const size_t lds_far = sizeof(float) * (64 * TOK_BMAX + D + (size_t)(TOK_THREADS / 64) * D + 64 + 6 * 16 + 4);
    const size_t lds = lds_near > lds_far ? lds_near : lds_far;   // <= 21 KiB
    hipLaunchKernelGGL(k_tok_part<D>, dim3(p.G * nsplit + p.nh * TOK_FB), dim3(TOK_THREADS), lds, st, p, part,
                       nsplit);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds_merge = sizeof(float) * (32 + (size_t)(TOK_MT / 64 + TOK_FB) * D);
    hipLaunchKernelGGL(k_tok_merge<D>, dim3(p.nh), dim3(TOK_MT), lds_merge, st, p, (const float*)part, nsplit);
    return hipGetLastError();
}

hipError_t launch_token(const KParams& p, float* part, hipStream_t st)
{
    const int nsplit = tok_splits(p.ns, p.W);
    switch (p.d) {
    case 8: return launch_two<8>(p, part, nsplit, st);
    case 16: return launch_two<16>(p, part, nsplit, st);
    case 32: return launch_two<32>(p, part, nsplit, st);
    case 64: return launch_two<64>(p, part, nsplit, st);
    case 128: return launch_two<128>(p, part, nsplit, st);
    case 256: return launch_two<256>(p, part, nsplit, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace swl
