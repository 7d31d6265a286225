// Far-field kernels: eviction scores, the running max / mass scan and the
// value accumulator.  cortiq-engine 0.8.51 src/gpu_wgpu/o1_batch.rs,
// o1b_far_e and o1b_far_commit, generalised from one sub-chunk to the S
// sub-chunks of a call: the score and value products of every sub-chunk run
// in parallel on MFMA (fp16 hi/lo splits, fp32 accuracy), and only the
// per-landmark recurrences (M and Z as scalars, Theta elementwise) walk the
// sub-chunks in order.
//
// Per sub-chunk s and landmark row (gh, b), with l_j the score of the key
// evicted by chunk row j (rows j0 <= j < k_s evict):
//   M'_s = max(M_{s-1}, max_j l_j);  R_s = 1 if M'_s == M_{s-1} else
//   exp(M_{s-1} - M'_s) (an empty field at -inf keeps R = 1 until its first
//   eviction, which then rescales the zero mass by exp(-inf) = 0);
//   E_sj = exp(l_j - M'_s);  Z_s = R_s Z_{s-1} + sum_j E_sj;
//   Theta_s = R_s Theta_{s-1} + sum_j E_sj v_evicted(j).
#include <type_traits>

#include "swl_internal.h"
#include "lanes.h"
#include "stages.h"

namespace swl {

typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int fkap(int v, int hf) { return (v >> 2) * 8 + hf * 4 + (v & 3); }

// fp32-accurate products on fp16 matrix cores, as in the attention kernel:
// x = hi + lo * 2^-11 (hi and the scaled remainder lo rounded to nearest), a
// product is hi*hi + (hi*lo + lo*hi) * 2^-11 with fp32 accumulation.
typedef _Float16 fhalf8 __attribute__((ext_vector_type(8)));
typedef unsigned int fu32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int fu32x2 __attribute__((ext_vector_type(2)));
constexpr float F_LO_UP = 2048.f;
constexpr float F_LO_DOWN = 1.f / 2048.f;

__device__ __forceinline__ floatx16 fmfma16(fu32x4 a, fu32x4 b, floatx16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(fhalf8, a),
                                                  __builtin_bit_cast(fhalf8, b), c, 0, 0, 0);
}
// (a, b) as an fp16 pair rounded to nearest, a in the low half
__device__ __forceinline__ unsigned fpk16n(float a, float b)
{
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(unsigned, h);
}
// hi/lo fp16 pairs of (a, b), both rounded to nearest (about 2^-22 error
// per product); lo scaled by 2^11 when SCALED.  a and b are pinned as
// rounded fp32 values first, so that a product in the caller cannot be
// contracted into one rounding of hi and not into the other.
template <bool SCALED>
__device__ __forceinline__ void fsplit(float a, float b, unsigned& hi, unsigned& lo)
{
    asm("" : "+v"(a), "+v"(b));
    hi = fpk16n(a, b);
    const float ra = a - (float)__builtin_bit_cast(_Float16, (unsigned short)(hi & 0xffffu));
    const float rb = b - (float)__builtin_bit_cast(_Float16, (unsigned short)(hi >> 16));
    lo = SCALED ? fpk16n(ra * F_LO_UP, rb * F_LO_UP) : fpk16n(ra, rb);
}
// 16-byte chunk c of row r of a [32][KD] fp16 tile sits at kswz(r, c): rows
// that one read touches start in different banks
template <int KD>
__device__ __forceinline__ int kswz(int r, int c)
{
    constexpr int CPR = KD / 8, RPB = KD >= 128 ? 1 : 128 / KD, M = (CPR < 16 ? CPR : 16) - 1;
    return c ^ ((r / RPB) & M);
}

// ---------------------------------------------------------------------------
// far_score: with l_j = scale <q~_{gh,b}, key evicted by row j>, per landmark
// row the local max mx = max_j l_j and E[s][gh*m+b][j] = exp(l_j - mx) (0
// for rows that do not evict), the local mass zl = sum_j E_j of the
// sub-chunk, and the accumulator increment TH[s][gh*m+b][t] = sum_j E_j
// v_evicted(j)[t].  Against the post-sub-chunk max M' every E_j is that
// times one factor, exp(mx - M') (far_scan), which the accumulator scan and
// the attention epilogue apply, so nothing here waits on the scan.
//
// One block per (group, run of `rl` consecutive sub-chunks, up to FS_RUN),
// or, in a launch of few runs, per (group, run, share of the landmark-row
// tiles) (fs_tsplit).  The block's waves take its tiles in turn; when there
// are waves to spare, two or four take each tile (all form its scores, each
// its share of the increments' columns), and when every tile has a wave its
// query halves stay in registers for the whole run.  The evicted keys of a
// sub-chunk are staged in LDS as fp16 hi/lo and its evicted values
// transposed as fp16 hi/lo; the loads for the next sub-chunk are in flight
// while the current one is multiplied.  Scores: MFMA C[j][hb] = K_e Q~^T on
// v_mfma_f32_32x32x16_f16 (three split products per k-step), which leaves a
// lane holding one landmark row's scores over 32 rows j; the max and mass
// over j are then in-lane sums plus one exchange between the lane halves,
// and E * 2^12 from those registers is the A operand of the increments'
// products C[hb][t] = E V_e (values times the sub-chunk's own power of two;
// both scaled back exactly).
//
// As the first launch of a call it also copies the call-start meta to
// p.meta_copy (block 0), which the later launches read, so that the last one
// can write the new meta, and, in a call without a far scan launch
// (p.vm_far), takes the value maxima (value_max_share) in FS_MIN_BLOCKS
// blocks per group of their own, after the working ones.
// ---------------------------------------------------------------------------
// eight waves; four at d = 256, where the query halves alone take 128 registers
template <int D>
constexpr int fs_threads() { return D > 128 ? 256 : 512; }

template <int D>
__global__ __launch_bounds__(fs_threads<D>()) void k_far_score(KParams p)
{
    constexpr int FS_THREADS = fs_threads<D>();
    constexpr int KD = D < 16 ? 16 : D;    // key width padded to whole k-steps
    constexpr int NS = KD / 16;
    constexpr int KH = 32 * KD;            // halves of one [32][KD] tile
    constexpr int NWV = FS_THREADS / 64;
    constexpr int NT = D >= 32 ? D / 32 : 1;   // 32-column tiles of the increments
    constexpr int VH = D * SUB;                // halves of one plane of the staged values
    // the evicted keys of a sub-chunk as fp16 hi/lo: rows j = 32 jt + r in
    // tile jt (hi at jt * 2 KH, lo KH further), zero for rows that do not
    // evict and for the columns past D
    __shared__ __align__(16) unsigned short ek[2 * 2 * KH];
    // the evicted values of a sub-chunk, transposed, as fp16 hi/lo times
    // the sub-chunk's power of two: column t holds the 64 rows j in eight
    // chunks of eight halves, chunk 2 (j / 16) + (j / 4) % 2 holding the rows
    // 16 (j / 16) + 4 ((j / 4) % 2) + {0 .. 3, 8 .. 11} in that order (the
    // rows of one k-step of the increments in one lane half), placed at
    // chunk c ^ ((t / 2) % 8) so that the columns one read touches start in
    // different banks; the lo plane VH halves further
    __shared__ __align__(16) unsigned short vt[2 * VH];
    __shared__ float vmw[NWV];             // per wave: largest |value| of the next sub-chunk
    typedef float v4 __attribute__((ext_vector_type(4)));
    constexpr int N = SUB * (KD / 4);      // 4-column pieces of the 64 rows
    constexpr int PT = (N + FS_THREADS - 1) / FS_THREADS;
    constexpr int NV = (SUB / 2) * (D / 4);   // (two rows) x (four columns) pieces of the values
    constexpr int PV = (NV + FS_THREADS - 1) / FS_THREADS;

    const int hm = p.H * p.m;
    const int rl = fs_run(p.S, p.G);
    const int nrun = fs_runs(p.S, p.G);
    const int ts = fs_tsplit(p.S, p.G, hm);
    // nrun * ts working blocks, then (taking the value maxima) FS_MIN_BLOCKS more
    const int nblk = nrun * ts + (p.vm_far ? FS_MIN_BLOCKS : 0);
    const int w = xcd_work_item(blockIdx.x, nblk * p.G);
    const int bi = w % nblk, g = w / nblk;
    const int run = bi / ts, tp = bi % ts;
    const int s_lo = min(run, nrun - 1) * rl, s_hi = min(p.S, s_lo + rl);
    const GMeta c = load_gmeta(p.meta, g, p.W);
    const int64_t nhm = (int64_t)p.nh * p.m;
    const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, ln = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nht = (hm + 31) / 32;
    // this block's landmark-row tiles [t_lo, t_hi) of the run's sub-chunks
    const int tpt = (nht + ts - 1) / ts;
    const int t_lo = min(tp * tpt, nht), t_hi = min(t_lo + tpt, nht);
    // with waves to spare, dup (2 or 4) waves take each tile: all of them
    // form its scores, and each forms its share of the increments' column
    // tiles (not at d = 256, whose four waves hold too many registers for
    // a second form of the increments)
    int dup = 1;
    while (D <= 128 && 2 * dup * (t_hi - t_lo) <= NWV && 2 * dup <= NT) dup *= 2;
    const int part = wave % dup;
    const bool resident = (t_hi - t_lo) * dup <= NWV;   // one landmark-row tile per wave at most

    // clamped unconditional loads of sub-chunk s's evicted keys (all in
    // flight at once), then their rows and columns selected at the store
    auto load_keys = [&](int s, v4 (&x)[PT]) {
        const int r0 = s * SUB, ks = min(SUB, p.T - r0);
#pragma unroll
        for (int u = 0; u < PT; ++u) {
            const int e = min(tid + u * FS_THREADS, N - 1);
            const int j = e / (KD / 4), c4 = min((e % (KD / 4)) * 4, D - 4);
            const int pos = max(c.len0 + r0 + min(j, ks - 1) - c.wg, 0);
            const float* ra = p.ring_k + ((int64_t)g * p.W + (c.head0 + min(pos, max(c.len0 - 1, 0))) % c.wg) * D;
            const float* ia = p.k + ((int64_t)max(pos - c.len0, 0) * p.G + g) * D;
            // a key from the call's rows takes the RoPE of its row on the way in
            const float* kt = (p.rope && pos >= c.len0) ? p.rope + (int64_t)(pos - c.len0) * D : nullptr;
            const float4 kx = rope4(pos < c.len0 ? ra : ia, kt, c4, D);
            x[u] = v4{kx.x, kx.y, kx.z, kx.w};
        }
    };
    auto store_keys = [&](int s, const v4 (&x)[PT], unsigned short* eb) {
        const int r0 = s * SUB, ks = min(SUB, p.T - r0);
        const int jlo = max(sub_meta(c, r0).j0, 0);
#pragma unroll
        for (int u = 0; u < PT; ++u) {
            const int e = tid + u * FS_THREADS;
            if (e < N) {
                const int j = e / (KD / 4), c4 = (e % (KD / 4)) * 4;
                const bool live = (j >= jlo) & (j < ks) & (c4 < D);
                unsigned h0, l0, h1, l1;
                fsplit<true>(live ? x[u].x : 0.f, live ? x[u].y : 0.f, h0, l0);
                fsplit<true>(live ? x[u].z : 0.f, live ? x[u].w : 0.f, h1, l1);
                const int jt = j >> 5, r = j & 31;
                unsigned short* t = eb + jt * 2 * KH + r * KD + kswz<KD>(r, c4 >> 3) * 8 + (c4 & 4);
                *reinterpret_cast<fu32x2*>(t) = fu32x2{h0, h1};
                *reinterpret_cast<fu32x2*>(t + KH) = fu32x2{l0, l1};
            }
        }
    };
    // the evicted values of sub-chunk s: clamped unconditional loads of
    // rows (2 jp, 2 jp + 1) x four columns per piece
    auto load_vals = [&](int s, v4 (&x)[PV][2]) {
        const int r0 = s * SUB, ks = min(SUB, p.T - r0);
#pragma unroll
        for (int u = 0; u < PV; ++u) {
            const int e = min(tid + u * FS_THREADS, NV - 1);
            const int jp = e / (D / 4), c4 = (e % (D / 4)) * 4;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int j = 2 * jp + r;
                const int pos = max(c.len0 + r0 + min(j, ks - 1) - c.wg, 0);
                const float* ra = p.ring_v + ((int64_t)g * p.W + (c.head0 + min(pos, max(c.len0 - 1, 0))) % c.wg) * D;
                const float* ia = p.v + ((int64_t)max(pos - c.len0, 0) * p.G + g) * D;
                x[u][r] = *reinterpret_cast<const v4*>((pos < c.len0 ? ra : ia) + c4);
            }
        }
    };
    // the largest |value| among this thread's pieces of rows that evict
    auto vals_max = [&](int s, const v4 (&x)[PV][2]) {
        const int r0 = s * SUB, ks = min(SUB, p.T - r0);
        const int jlo = max(sub_meta(c, r0).j0, 0);
        float mv = 0.f;
#pragma unroll
        for (int u = 0; u < PV; ++u) {
            const int e = tid + u * FS_THREADS;
            const int jp = e / (D / 4);
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int j = 2 * jp + r;
                const bool live = (e < NV) & (j >= jlo) & (j < ks);
                const float a = fmaxf(fmaxf(fabsf(x[u][r].x), fabsf(x[u][r].y)), fmaxf(fabsf(x[u][r].z), fabsf(x[u][r].w)));
                mv = fmaxf(mv, live ? a : 0.f);
            }
        }
        return mv;
    };
    // the pieces into vt, times 2^vexp, zero for rows that do not evict
    auto store_vals = [&](int s, const v4 (&x)[PV][2], int vexp) {
        const int r0 = s * SUB, ks = min(SUB, p.T - r0);
        const int jlo = max(sub_meta(c, r0).j0, 0);
#pragma unroll
        for (int u = 0; u < PV; ++u) {
            const int e = tid + u * FS_THREADS;
            if (e < NV) {
                const int jp = e / (D / 4), c4 = (e % (D / 4)) * 4, j = 2 * jp;
                const bool l0 = (j >= jlo) & (j < ks), l1 = (j + 1 >= jlo) & (j + 1 < ks);
                const int ch = 2 * (j >> 4) + ((j >> 2) & 1), el = ((j >> 3) & 1) * 4 + (j & 3);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int t = c4 + q;
                    unsigned hi, lo;
                    fsplit<false>(l0 ? ldexpf(x[u][0][q], vexp) : 0.f, l1 ? ldexpf(x[u][1][q], vexp) : 0.f, hi, lo);
                    const int at = t * SUB + ((ch ^ ((t >> 1) & 7)) << 3) + el;
                    *reinterpret_cast<unsigned*>(vt + at) = hi;
                    *reinterpret_cast<unsigned*>(vt + VH + at) = lo;
                }
            }
        }
    };
    // landmark query halves of tile ht: q~[hb][16 st + 8 hf + e] times
    // scale * log2 e, so that the scores come out in base 2
    fu32x4 qah[NS], qal[NS];
    auto fetch_q = [&](int ht, float4 (&x)[NS][2]) {
        const int hb_a = ht * 32 + ln;   // A row of this lane
        const float* qr = p.q_tilde + ((int64_t)g * hm + min(hb_a, hm - 1)) * D;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const int d0 = 16 * st + 8 * hf;
            x[st][0] = x[st][1] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (d0 < D) {
                x[st][0] = *reinterpret_cast<const float4*>(qr + d0);
                x[st][1] = *reinterpret_cast<const float4*>(qr + d0 + 4);
            }
        }
    };
    auto split_q = [&](const float4 (&x)[NS][2]) {
        const float qs = p.scale * 1.4426950408889634f;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            unsigned h[4], l[4];
            fsplit<true>(x[st][0].x * qs, x[st][0].y * qs, h[0], l[0]);
            fsplit<true>(x[st][0].z * qs, x[st][0].w * qs, h[1], l[1]);
            fsplit<true>(x[st][1].x * qs, x[st][1].y * qs, h[2], l[2]);
            fsplit<true>(x[st][1].z * qs, x[st][1].w * qs, h[3], l[3]);
            qah[st] = fu32x4{h[0], h[1], h[2], h[3]};
            qal[st] = fu32x4{l[0], l[1], l[2], l[3]};
        }
    };
    auto load_q = [&](int ht) {
        float4 x[NS][2];
        fetch_q(ht, x);
        split_q(x);
    };

    if (blockIdx.x == 0 && tid < 4 * p.G) p.meta_copy[tid] = p.meta[tid];
    if (bi >= nrun * ts) {
        // a block for the value maxima only (uniform over the block): share
        // bi - nrun * ts of FS_MIN_BLOCKS, so that the working blocks do not
        // wait on those loads
        __shared__ float vred[FS_THREADS / 64];
        value_max_share<D, FS_THREADS>(p, c, g, bi - nrun * ts, FS_MIN_BLOCKS, vred);
        return;
    }
    // the query halves' loads go out first, beside the keys' and values',
    // and are split after them
    const bool qpre = resident && wave < (t_hi - t_lo) * dup;   // (uniform)
    float4 qx[NS][2];
    if (qpre) fetch_q(t_lo + wave / dup, qx);
    v4 xk[PT];
    v4 xv[PV][2];
    {
        load_keys(s_lo, xk);
        load_vals(s_lo, xv);
        const float mv = wmax(vals_max(s_lo, xv));
        if (lane == 0) vmw[wave] = mv;
    }
    if (qpre) split_q(qx);
#pragma unroll 1
    for (int s = s_lo; s < s_hi; ++s) {
        __syncthreads();   // ek and vt are no longer read; vmw holds sub-chunk s's wave maxima
        store_keys(s, xk, ek);
        // the increments take the values times a power of two of their own
        // (the result is scaled back exactly), so that small values keep
        // their remainders far above fp16's floor
        float vm = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NWV; ++w2) vm = fmaxf(vm, vmw[w2]);
        const int vexp = __builtin_amdgcn_readfirstlane(value_exp_of(vm));
        store_vals(s, xv, vexp);
        __syncthreads();   // ek and vt hold sub-chunk s
        const bool next = s + 1 < s_hi;
        if (next) {
            load_keys(s + 1, xk);
            load_vals(s + 1, xv);
        }

        const int r0 = s * SUB, ks = min(SUB, p.T - r0);
        const int jlo = max(sub_meta(c, r0).j0, 0);
        float* L = p.E + ((int64_t)s * nhm + (int64_t)g * hm) * SUB;
        float* MX = p.Ms + (int64_t)s * nhm + (int64_t)g * hm;   // local max (the scan overwrites)
        float* ZL = p.Rs + (int64_t)s * nhm + (int64_t)g * hm;   // local mass (the scan overwrites)
        float* TI = p.TH + ((int64_t)s * nhm + (int64_t)g * hm) * D;   // the increments
        for (int ht = t_lo + wave / dup; ht < t_hi; ht += NWV / dup) {
            if (!resident) load_q(ht);
            // C[j][hb] = K_e Q~^T: the keys are the A operand, so that a
            // lane ends with one landmark row's scores over 32 rows j; both
            // 32-row tiles of keys in one k-step loop: each step's query
            // halves feed six products on four accumulators, and the LDS
            // reads run two steps ahead of their products
            floatx16 sh[2], sx[2];
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    sh[jt][v] = 0.f;
                    sx[jt][v] = 0.f;
                }
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const int ck = kswz<KD>(ln, 2 * st + hf) * 8;
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) {
                    const unsigned short* kr = ek + jt * 2 * KH + ln * KD + ck;
                    const fu32x4 bh = *reinterpret_cast<const fu32x4*>(kr);
                    const fu32x4 bl = *reinterpret_cast<const fu32x4*>(kr + KH);
                    sh[jt] = fmfma16(bh, qah[st], sh[jt]);
                    sx[jt] = fmfma16(bl, qah[st], sx[jt]);
                    sx[jt] = fmfma16(bh, qal[st], sx[jt]);
                }
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
                if (st + 2 < NS) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            }
            // lane holds landmark row hb = ht*32 + ln, rows j = jt*32 +
            // kappa(v, hf); scores and their max in base 2 (the max is
            // stored in natural units, as the state keeps M)
            floatx16 acc[2];
            float m2 = -INFINITY;
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int j = jt * 32 + fkap(v, hf);
                    const float l = (j >= jlo && j < ks) ? fmaf(sx[jt][v], F_LO_DOWN, sh[jt][v]) : -INFINITY;
                    acc[jt][v] = l;
                    m2 = fmaxf(m2, l);
                }
            const float mx = pair_max<5>(m2);   // with the other half's 32 rows
            float z = 0.f;
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    // exp(l - mx) as 2^(l2 - mx2): 0 for rows that do not evict (and
                    // when none does; results below 2^-126 flush to 0)
                    acc[jt][v] = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(acc[jt][v] - mx);
                    z += acc[jt][v];
                }
            z = pair_sum<5>(z);
            const int hb = ht * 32 + ln;
            if (hb < hm && part == 0) {
#pragma unroll
                for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<float4*>(L + (int64_t)hb * SUB + jt * 32 + q * 8 + hf * 4) =
                            make_float4(acc[jt][4 * q], acc[jt][4 * q + 1], acc[jt][4 * q + 2], acc[jt][4 * q + 3]);
                if (hf == 0) {
                    MX[hb] = mx * 0.6931471805599453f;   // ln 2
                    ZL[hb] = z;
                }
            }
            // the increments TI[hb][t] = sum_j E_hb,j v_j[t] against the
            // local max (the accumulator scan applies fac_s): C[hb][t] with
            // E * 2^12 as the A operand straight from the registers above,
            // k-step kk taking rows j = 16 kk + 8 (i / 4) + 4 hf + i % 4 of
            // the lane's eight (i = 0 .. 7), the order of vt's chunks
            fu32x4 eh[4], el[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                unsigned h[4], l[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    fsplit<false>(acc[kk >> 1][(kk & 1) * 8 + 2 * q] * 4096.f,
                                  acc[kk >> 1][(kk & 1) * 8 + 2 * q + 1] * 4096.f, h[q], l[q]);
                eh[kk] = fu32x4{h[0], h[1], h[2], h[3]};
                el[kk] = fu32x4{l[0], l[1], l[2], l[3]};
            }
            // this wave's column tiles [c_lo, c_hi), NCC at a time (k-step
            // outer, tiles inner: consecutive products go to different
            // accumulators)
            const int c_lo = part * (NT / dup), c_hi = c_lo + NT / dup;
            auto incr = [&](auto ncc) {
                constexpr int NCC = decltype(ncc)::value;
#pragma unroll
                for (int t0 = 0; t0 < NT; t0 += NCC) {
                    if (t0 < c_lo || t0 >= c_hi) continue;   // (uniform)
                    floatx16 ad[NCC];
#pragma unroll
                    for (int tt = 0; tt < NCC; ++tt)
#pragma unroll
                        for (int v = 0; v < 16; ++v) ad[tt][v] = 0.f;
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                        for (int tt = 0; tt < NCC; ++tt) {
                            const int t = min((t0 + tt) * 32 + ln, D - 1);
                            const int at = t * SUB + (((2 * kk + hf) ^ ((t >> 1) & 7)) << 3);
                            const fu32x4 vh = *reinterpret_cast<const fu32x4*>(vt + at);
                            const fu32x4 vl = *reinterpret_cast<const fu32x4*>(vt + VH + at);
                            ad[tt] = fmfma16(eh[kk], vh, ad[tt]);
                            ad[tt] = fmfma16(eh[kk], vl, ad[tt]);
                            ad[tt] = fmfma16(el[kk], vh, ad[tt]);
                        }
                    }
                    // lane holds rows hb = ht*32 + kappa(v, hf), columns t = (t0 + tt)*32 + ln
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int hbo = ht * 32 + fkap(v, hf);
                        if (hbo < hm) {
#pragma unroll
                            for (int tt = 0; tt < NCC; ++tt) {
                                const int t = (t0 + tt) * 32 + ln;
                                if (t < D) TI[(int64_t)hbo * D + t] = ldexpf(ad[tt][v], -12 - vexp);
                            }
                        }
                    }
                }
            };
            constexpr int NC = NT < 2 ? NT : 2;
            if (D > 128 || NT / dup >= NC) incr(std::integral_constant<int, NC>{});
            else if constexpr (D <= 128) incr(std::integral_constant<int, 1>{});
        }
        if (next) {
            const float mv = wmax(vals_max(s + 1, xv));
            if (lane == 0) vmw[wave] = mv;
        }
    }
}

// ---------------------------------------------------------------------------
template <int D>
static void launch_fs(const KParams& p, hipStream_t st)
{
    const int hm = p.H * p.m;
    const int nblk = fs_runs(p.S, p.G) * fs_tsplit(p.S, p.G, hm) + (p.vm_far ? FS_MIN_BLOCKS : 0);
    hipLaunchKernelGGL(k_far_score<D>, dim3(nblk * p.G), dim3(fs_threads<D>()), 0, st,
                       p);
}

hipError_t launch_far_score(const KParams& p, hipStream_t st)
{
    switch (p.d) {
    case 8: launch_fs<8>(p, st); break;
    case 16: launch_fs<16>(p, st); break;
    case 32: launch_fs<32>(p, st); break;
    case 64: launch_fs<64>(p, st); break;
    case 128: launch_fs<128>(p, st); break;
    case 256: launch_fs<256>(p, st); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The far scan in a launch of its own (stages.h, mz_scan_row): a block of
// eight waves takes eight consecutive landmark rows, whose values of a
// sub-chunk sit side by side in each plane.  It reads the rows' (mx, zl)
// into LDS in 32-byte runs, a wave scans each row from there, and the
// results go back to the planes the same way.  (Read straight from the
// planes, each lane's sub-chunks are a plane row apart: one 32-byte sector
// moved per value.)  With `vm` the launch also takes the value maxima that
// the key tiles and the far readout scale by: p.vm_n blocks per group after
// the scan's (value_max_share), which the scan blocks do not wait for.
constexpr int FSC_ROWS = 8;
constexpr int FSC_SP = PASS_SUBS + 1;   // LDS row stride, odd: the rows of one sub-chunk in different banks

template <int D>
__global__ __launch_bounds__(64 * FSC_ROWS) void k_far_scan(KParams p, int nscan)
{
    if ((int)blockIdx.x >= nscan) {
        // the value maxima: p.vm_n blocks per group, as far_score takes them
        // in a call without this launch
        __shared__ float vred[FSC_ROWS];
        const int v = (int)blockIdx.x - nscan, g = v / p.vm_n;
        value_max_share<D, 64 * FSC_ROWS>(p, load_gmeta(p.meta, g, p.W), g, v % p.vm_n, p.vm_n, vred);
        return;
    }
    __shared__ float lm[FSC_ROWS * FSC_SP], lz[FSC_ROWS * FSC_SP], lt[FSC_ROWS * FSC_SP], lf[FSC_ROWS * FSC_SP];
    const int64_t nhm = (int64_t)p.nh * p.m;
    const int64_t ghb0 = (int64_t)blockIdx.x * FSC_ROWS;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    constexpr int NT = 64 * FSC_ROWS;
    constexpr int PER = PASS_SUBS * FSC_ROWS / NT;   // (sub-chunk, row) elements per thread
    // element i: sub-chunk i / FSC_ROWS, row i % FSC_ROWS
    {
        float a[PER], z[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + k * NT, s = min(i / FSC_ROWS, p.S - 1);
            const int64_t row = min(ghb0 + i % FSC_ROWS, nhm - 1);
            a[k] = p.Ms[(int64_t)s * nhm + row];
            z[k] = p.Rs[(int64_t)s * nhm + row];
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + k * NT, s = i / FSC_ROWS, r = i % FSC_ROWS;
            lm[r * FSC_SP + s] = a[k];
            lz[r * FSC_SP + s] = z[k];
        }
    }
    __syncthreads();
    const int64_t ghb = ghb0 + w;
    if (ghb < nhm) {
        float* const m = lm + w * FSC_SP;
        float* const zr = lz + w * FSC_SP;
        float* const t = lt + w * FSC_SP;
        float* const f = lf + w * FSC_SP;
        mz_scan_row(
            p, ghb, lane, [&](int s) { return make_float2(m[s], zr[s]); },
            [&](int s, float Mn, float R, float Z, float fac) {
                if (s < p.S) {
                    m[s] = Mn;
                    zr[s] = R;
                    f[s] = fac;
                }
                t[s] = Z;
            });
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = tid + k * NT, s = i / FSC_ROWS, r = i % FSC_ROWS;
        const int64_t row = ghb0 + r;
        if (s < p.S && row < nhm) {
            const int64_t at = (int64_t)s * nhm + row;
            p.Ms[at] = lm[r * FSC_SP + s];
            p.Rs[at] = lz[r * FSC_SP + s];
            p.TZ[at] = lt[r * FSC_SP + s];
            p.FAC[at] = lf[r * FSC_SP + s];
        }
    }
    if (tid < FSC_ROWS && ghb0 + tid < nhm) p.TZ[(int64_t)p.S * nhm + ghb0 + tid] = lt[tid * FSC_SP + p.S];
}

template <int D>
static void launch_fsc(const KParams& p, bool vm, hipStream_t st)
{
    const int64_t n = ((int64_t)p.nh * p.m + FSC_ROWS - 1) / FSC_ROWS;
    const int64_t nv = vm ? (int64_t)p.vm_n * p.G : 0;
    hipLaunchKernelGGL(k_far_scan<D>, dim3((unsigned)(n + nv)), dim3(64 * FSC_ROWS), 0, st, p, (int)n);
}

hipError_t launch_far_scan(const KParams& p, bool vm, hipStream_t st)
{
    switch (p.d) {
    case 8: launch_fsc<8>(p, vm, st); break;
    case 16: launch_fsc<16>(p, vm, st); break;
    case 32: launch_fsc<32>(p, vm, st); break;
    case 64: launch_fsc<64>(p, vm, st); break;
    case 128: launch_fsc<128>(p, vm, st); break;
    case 256: launch_fsc<256>(p, vm, st); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace swl
