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
#include "swl_internal.h"
#include "lanes.h"

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
// for rows that do not evict) and the local mass zl = sum_j E_j of the
// sub-chunk.  Against the post-sub-chunk max M' every E_j is that times one
// factor, exp(mx - M') (far_scan), which the accumulator scan and the
// attention epilogue apply.  One block per (group, run of
// `rl` consecutive sub-chunks, up to FS_RUN); wave w of the block's NWV takes
// landmark-row tiles w, w + NWV, ..., and when a group has at most NWV of
// them its tile's query halves stay in registers for the whole run.  The evicted keys of a
// sub-chunk are staged in LDS as fp16 hi/lo, double-buffered: the loads for
// the next sub-chunk are in flight while the current one is multiplied.
// MFMA C[hb][j] = Q~ K_e^T on v_mfma_f32_32x32x16_f16 (three split products
// per k-step; lane (row, hf) holds columns 16 st + 8 hf .. +7 of its row).
//
// As the first launch of a call it also (a) copies the call-start meta to
// p.meta_copy (block 0), which the later launches read, so that the last one
// can write the new meta, and (b) takes the largest |value| of an equal share
// of its group's value rows -- the sinks, the window at the call's start and
// the call's rows -- into p.vmax[g][run]: the value products of the call
// (key tiles, accumulator increments) scale their fp16 splits by the
// group's maximum (value_exp).
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
    // two buffers of the evicted keys of a sub-chunk as fp16 hi/lo: rows
    // j = 32 jt + r in tile jt (hi at jt * 2 KH, lo KH further), zero for
    // rows that do not evict and for the columns past D
    __shared__ __align__(16) unsigned short ek[2][2 * 2 * KH];
    typedef float v4 __attribute__((ext_vector_type(4)));
    constexpr int N = SUB * (KD / 4);      // 4-column pieces of the 64 rows
    constexpr int PT = (N + FS_THREADS - 1) / FS_THREADS;

    const int rl = fs_run(p.S, p.G);
    const int nrun = fs_runs(p.S, p.G);
    const int nblk = fs_blocks_per_group(p.S, p.G);   // nrun, or more for short calls
    const int w = xcd_work_item(blockIdx.x, nblk * p.G);
    const int run = w % nblk, g = w / nblk;
    const int s_lo = min(run, nrun - 1) * rl, s_hi = min(p.S, s_lo + rl);
    const GMeta c = load_gmeta(p.meta, g, p.W);
    const int hm = p.H * p.m;
    const int64_t nhm = (int64_t)p.nh * p.m;
    const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, ln = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nht = (hm + 31) / 32;
    const bool resident = nht <= NWV;      // one landmark-row tile per wave at most

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
    // landmark query halves of tile ht: q~[hb][16 st + 8 hf + e] times
    // scale * log2 e, so that the scores come out in base 2
    fu32x4 qah[NS], qal[NS];
    auto load_q = [&](int ht) {
        const float qs = p.scale * 1.4426950408889634f;
        const int hb_a = ht * 32 + ln;   // A row of this lane
        const float* qr = p.q_tilde + ((int64_t)g * hm + min(hb_a, hm - 1)) * D;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const int d0 = 16 * st + 8 * hf;
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x;
            if (d0 < D) {
                x = *reinterpret_cast<const float4*>(qr + d0);
                y = *reinterpret_cast<const float4*>(qr + d0 + 4);
            }
            unsigned h[4], l[4];
            fsplit<true>(x.x * qs, x.y * qs, h[0], l[0]);
            fsplit<true>(x.z * qs, x.w * qs, h[1], l[1]);
            fsplit<true>(y.x * qs, y.y * qs, h[2], l[2]);
            fsplit<true>(y.z * qs, y.w * qs, h[3], l[3]);
            qah[st] = fu32x4{h[0], h[1], h[2], h[3]};
            qal[st] = fu32x4{l[0], l[1], l[2], l[3]};
        }
    };

    if (blockIdx.x == 0 && tid < 4 * p.G) p.meta_copy[tid] = p.meta[tid];
    {
        v4 x[PT];
        load_keys(s_lo, x);
        // the largest |value| of this block's share of the group's value rows
        // (its loads go out beside the first sub-chunk's keys)
        {
            constexpr int LPR = D / 4 < 64 ? D / 4 : 64;   // lanes per row (d <= 256: one float4 each)
            constexpr int RPB = FS_THREADS / LPR;           // rows per step
            constexpr int U = 4;                            // steps in flight
            const int64_t n = (int64_t)p.ns + c.len0 + p.T;
            const int r_lo = (int)(n * run / nblk), r_hi = (int)(n * (run + 1) / nblk);
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
            __shared__ float vred[FS_THREADS / 64];
            if (lane == 0) vred[wave] = mx;
            __syncthreads();
            if (tid == 0) {
                float b = 0.f;
#pragma unroll
                for (int w2 = 0; w2 < FS_THREADS / 64; ++w2) b = fmaxf(b, vred[w2]);
                p.vmax[(int64_t)g * VM_SLOTS + run] = b;
            }
        }
        if (run >= nrun) return;   // a block for the value maxima only (uniform over the block)
        store_keys(s_lo, x, ek[0]);
    }
    if (resident && wave < nht) load_q(wave);
#pragma unroll 1
    for (int s = s_lo; s < s_hi; ++s) {
        const int buf = (s - s_lo) & 1;
        __syncthreads();   // ek[buf] holds sub-chunk s; ek[buf ^ 1] is no longer read
        v4 xn[PT];
        const bool next = s + 1 < s_hi;
        if (next) load_keys(s + 1, xn);

        const int r0 = s * SUB, ks = min(SUB, p.T - r0);
        const int jlo = max(sub_meta(c, r0).j0, 0);
        float* L = p.E + ((int64_t)s * nhm + (int64_t)g * hm) * SUB;
        float* MX = p.Ms + (int64_t)s * nhm + (int64_t)g * hm;   // local max (the scan overwrites)
        float* ZL = p.Rs + (int64_t)s * nhm + (int64_t)g * hm;   // local mass (the scan overwrites)
        const unsigned short* eb = ek[buf];
        for (int ht = wave; ht < nht; ht += NWV) {
            if (!resident) load_q(ht);
            // both 32-row tiles of evicted keys in one k-step loop: each
            // step's query halves feed six products on four accumulators,
            // and the LDS reads run two steps ahead of their products
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
                    const unsigned short* kr = eb + jt * 2 * KH + ln * KD + ck;
                    const fu32x4 bh = *reinterpret_cast<const fu32x4*>(kr);
                    const fu32x4 bl = *reinterpret_cast<const fu32x4*>(kr + KH);
                    sh[jt] = fmfma16(qah[st], bh, sh[jt]);
                    sx[jt] = fmfma16(qah[st], bl, sx[jt]);
                    sx[jt] = fmfma16(qal[st], bh, sx[jt]);
                }
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
                if (st + 2 < NS) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            }
            floatx16 acc[2];
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[jt][v] = fmaf(sx[jt][v], F_LO_DOWN, sh[jt][v]);
            // lane holds rows hb = ht*32 + kappa(v, hf), columns j = jt*32 + ln;
            // scores and their max in base 2 (the max is stored in natural
            // units, as the state keeps M)
            float mx[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                float m2 = -INFINITY;
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) {
                    const int j = jt * 32 + ln;
                    const float l = (j >= jlo && j < ks) ? acc[jt][v] : -INFINITY;
                    acc[jt][v] = l;
                    m2 = fmaxf(m2, l);
                }
                mx[v] = max32(m2);   // over the 32 evicting rows j of this lane half
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int hb = ht * 32 + fkap(v, hf);
                float z = 0.f;
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) {
                    // exp(l - mx) as 2^(l2 - mx2): 0 for rows that do not evict (and
                    // when none does; results below 2^-126 flush to 0)
                    acc[jt][v] = mx[v] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(acc[jt][v] - mx[v]);
                    z += acc[jt][v];
                }
                z = sum32(z);
                if (hb < hm) {
#pragma unroll
                    for (int jt = 0; jt < 2; ++jt) L[(int64_t)hb * SUB + jt * 32 + ln] = acc[jt][v];
                    if (ln == 0) {
                        MX[hb] = mx[v] * 0.6931471805599453f;   // ln 2
                        ZL[hb] = z;
                    }
                }
            }
        }
        if (next) store_keys(s + 1, xn, ek[buf ^ 1]);
    }
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

// One wave per landmark row; lane l takes sub-chunks MZ_PER l .. MZ_PER l +
// MZ_PER - 1 (MZ_PER = PASS_SUBS / 64, so S <= PASS_SUBS):
// the merge of each lane's run, an exclusive scan of the runs over the wave,
// then every lane applies the recurrence above to its own sub-chunks from
// the state before them (so M'_s and R_s are exactly the serial ones and Z
// differs from the serial sum only in rounding order).
constexpr int MZ_PER = PASS_SUBS / 64;

__device__ __forceinline__ void mz_scan_body(const KParams& p, int64_t bid)
{
    const int64_t nhm = (int64_t)p.nh * p.m;
    const int lane = threadIdx.x & 63;
    const int64_t ghb = bid * 4 + (threadIdx.x >> 6);
    if (ghb >= nhm) return;   // (uniform over the wave)
    const int64_t gh = ghb / p.m, b = ghb % p.m;
    float mx[MZ_PER], zl[MZ_PER];
#pragma unroll
    for (int k = 0; k < MZ_PER; ++k) {
        const int s = min(MZ_PER * lane + k, p.S - 1);
        mx[k] = p.Ms[(int64_t)s * nhm + ghb];
        zl[k] = p.Rs[(int64_t)s * nhm + ghb];
        if (MZ_PER * lane + k >= p.S) mx[k] = -INFINITY;   // past the last sub-chunk: empty
    }
    MZ run = {-INFINITY, 0.f};
#pragma unroll
    for (int k = 0; k < MZ_PER; ++k) run = mz_merge(run, MZ{mx[k], zl[k]});
    // inclusive scan over the lanes, then shift to the exclusive prefix
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const MZ o = {__shfl_up(run.M, d, 64), __shfl_up(run.Z, d, 64)};
        if (lane >= d) run = mz_merge(o, run);
    }
    MZ pre = {__shfl_up(run.M, 1, 64), __shfl_up(run.Z, 1, 64)};
    if (lane == 0) pre = {-INFINITY, 0.f};
    // the committed state before the call, then this lane's sub-chunks
    MZ st = mz_merge(MZ{p.mz[gh * 2 * p.m + b], p.mz[gh * 2 * p.m + p.m + b]}, pre);
    float M = st.M, Z = st.Z;
#pragma unroll
    for (int k = 0; k < MZ_PER; ++k) {
        const int s = MZ_PER * lane + k;
        if (s < p.S) {
            const float Mn = fmaxf(M, mx[k]);
            const float R = (Mn == M) ? 1.0f : expf(M - Mn);
            const int64_t at = (int64_t)s * nhm + ghb;
            const float fac = mx[k] == -INFINITY ? 0.f : expf(mx[k] - Mn);
            p.Ms[at] = Mn;
            p.Rs[at] = R;
            p.TZ[at] = Z;
            p.FAC[at] = fac;
            Z = R * Z + zl[k] * fac;
            M = Mn;
            // the mass after the last sub-chunk, which a commit stores: a call
            // that resumes from the committed state then carries this value
            if (s == p.S - 1) p.TZ[(int64_t)p.S * nhm + ghb] = Z;
        }
    }
}

// ---------------------------------------------------------------------------
// dtheta: per (sub-chunk, group): TH[s][gh*m+b][t] = sum_j E_bj
// v_evicted(j)[t] with far_score's E (against the sub-chunk's own max, so
// it needs nothing from the far scan; the accumulator scan applies fac_s)
// on fp16 MFMA with hi/lo splits (C[b][t]; each lane holds rows hf*32 .. +31
// of its E row, and k-step st takes rows 32 hf + 8 st .. +7).  E is scaled by 2^12 and the values by the pass's
// power of two (value_exp) before the split, so that the fp16 remainders of
// small values stay far above their absolute floor and large values stay in
// fp16 range; the result is scaled back exactly.  The evicted values are
// staged in LDS transposed.
// ---------------------------------------------------------------------------
template <int DV>
__device__ __forceinline__ void dtheta_body(const KParams& p, int64_t bid)
{
    constexpr int NT = DV >= 32 ? DV / 32 : 1;   // 32-column output tiles
    // the evicted values transposed, fp16 hi/lo: row t holds the 64 rows j
    // (chunk c = rows 8c .. 8c+7 at chunk c ^ ((t >> 1) & 7)), zero for rows
    // that do not evict
    constexpr int VH = DV * SUB;
    __shared__ __align__(16) unsigned short vt[2 * VH];
    const int w = (int)bid;
    const int s = w % p.S, g = w / p.S;
    const int r0 = s * SUB;
    const int ks = min(SUB, p.T - r0);
    const GMeta c = load_gmeta(p.meta, g, p.W);
    const SubMeta sm = sub_meta(c, r0);
    const int jlo = max(sm.j0, 0);
    const int hm = p.H * p.m;
    const int64_t nhm = (int64_t)p.nh * p.m;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, ln = lane & 31;
    const int64_t row0 = (int64_t)s * nhm + (int64_t)g * hm;   // landmark row (s, g*H*m)
    const int nht = (hm + 31) / 32;
    // this lane's E row of landmark-row tile ht (zero past hm)
    auto load_e = [&](int ht, float (&e)[32]) {
        const int hb = ht * 32 + ln;
        const bool rv = hb < hm;
        const float* Lr = p.E + (row0 + min(hb, hm - 1)) * SUB + hf * 32;
#pragma unroll
        for (int k = 0; k < 32; k += 4) {
            const float4 x = *reinterpret_cast<const float4*>(Lr + k);
            e[k] = rv ? x.x : 0.f; e[k + 1] = rv ? x.y : 0.f;
            e[k + 2] = rv ? x.z : 0.f; e[k + 3] = rv ? x.w : 0.f;
        }
    };
    // the wave's first tile's E rows go out before the values' staging
    float e0[32];
    if (wave < nht) load_e(wave, e0);
    const int vexp = value_exp(p, g);   // the values enter the split times 2^vexp
    {
        // units of two rows (2 jp, 2 jp + 1) x four columns: clamped
        // unconditional loads, then per column one fp16 pair of each half
        typedef float v4 __attribute__((ext_vector_type(4)));
        constexpr int N = (SUB / 2) * (DV / 4);
        constexpr int PT = (N + 255) / 256;
        v4 x[PT][2];
#pragma unroll
        for (int u = 0; u < PT; ++u) {
            const int e = min(tid + u * 256, N - 1);
            const int jp = e / (DV / 4), c4 = (e % (DV / 4)) * 4;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int j = 2 * jp + r;
                const int pos = max(c.len0 + r0 + min(j, ks - 1) - c.wg, 0);
                const float* ra = p.ring_v + ((int64_t)g * p.W + (c.head0 + min(pos, max(c.len0 - 1, 0))) % c.wg) * DV;
                const float* ia = p.v + ((int64_t)max(pos - c.len0, 0) * p.G + g) * DV;
                x[u][r] = *reinterpret_cast<const v4*>((pos < c.len0 ? ra : ia) + c4);
            }
        }
#pragma unroll
        for (int u = 0; u < PT; ++u) {
            const int e = tid + u * 256;
            if (e < N) {
                const int jp = e / (DV / 4), c4 = (e % (DV / 4)) * 4;
                const bool l0 = (2 * jp >= jlo) & (2 * jp < ks), l1 = (2 * jp + 1 >= jlo) & (2 * jp + 1 < ks);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int t = c4 + q;
                    unsigned hi, lo;
                    fsplit<false>(l0 ? ldexpf(x[u][0][q], vexp) : 0.f, l1 ? ldexpf(x[u][1][q], vexp) : 0.f, hi, lo);
                    const int at = t * SUB + (((jp >> 2) ^ ((t >> 1) & 7)) << 3) + ((2 * jp) & 7);
                    *reinterpret_cast<unsigned*>(vt + at) = hi;
                    *reinterpret_cast<unsigned*>(vt + VH + at) = lo;
                }
            }
        }
    }
    __syncthreads();
    auto tile = [&](int ht, const float (&e)[32]) {
        // E * 2^12 as fp16 halves: k-step st takes rows j = 32 hf + 8 st + e
        // of this lane's landmark row (its own e[8 st + e])
        fu32x4 eh[4], el[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            unsigned h[4], l[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                fsplit<false>(e[8 * st + 2 * q] * 4096.f, e[8 * st + 2 * q + 1] * 4096.f, h[q], l[q]);
            eh[st] = fu32x4{h[0], h[1], h[2], h[3]};
            el[st] = fu32x4{l[0], l[1], l[2], l[3]};
        }
        // k-step outer, column tiles inner: consecutive products go to
        // different accumulators, and the LDS reads run two steps ahead
        floatx16 acc[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[tt][v] = 0.f;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int t = min(tt * 32 + ln, DV - 1);
                const int at = t * SUB + (((4 * hf + st) ^ ((t >> 1) & 7)) << 3);
                const fu32x4 vh = *reinterpret_cast<const fu32x4*>(vt + at);
                const fu32x4 vl = *reinterpret_cast<const fu32x4*>(vt + VH + at);
                acc[tt] = fmfma16(eh[st], vh, acc[tt]);
                acc[tt] = fmfma16(eh[st], vl, acc[tt]);
                acc[tt] = fmfma16(el[st], vh, acc[tt]);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int k = 0; k < 4 * NT; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
            if (k + 2 < 4 * NT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[tt][v] = ldexpf(acc[tt][v], -12 - vexp);
        // lane holds rows hb = ht*32 + kappa(v, hf), columns t = tt*32 + ln
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int hbo = ht * 32 + fkap(v, hf);
            if (hbo < hm) {
                float* out = p.TH + (row0 + hbo) * DV;
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const int t = tt * 32 + ln;
                    if (t < DV) out[t] = acc[tt][v];
                }
            }
        }
    };
    if (wave < nht) tile(wave, e0);
    for (int ht = wave + 4; ht < nht; ht += 4) {
        float e[32];
        load_e(ht, e);
        tile(ht, e);
    }
}

// ---------------------------------------------------------------------------
template <int D>
static void launch_fs(const KParams& p, hipStream_t st)
{
    hipLaunchKernelGGL(k_far_score<D>, dim3(fs_blocks_per_group(p.S, p.G) * p.G), dim3(fs_threads<D>()), 0, st,
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

// The far scan (one wave per landmark row, four per block) and the
// accumulator increments (one block per (sub-chunk, group), XCD-ordered) in
// one launch: the increments take far_score's E as it is, so neither waits
// for the other.
template <int DV>
__global__ __launch_bounds__(256) void k_scan_dtheta(KParams p, int nmz)
{
    if ((int)blockIdx.x < nmz) mz_scan_body(p, blockIdx.x);
    else dtheta_body<DV>(p, xcd_work_item((int)blockIdx.x - nmz, p.S * p.G));
}

template <int DV>
static void launch_sd(const KParams& p, hipStream_t st)
{
    const int nmz = (int)(((int64_t)p.nh * p.m + 3) / 4);
    hipLaunchKernelGGL(k_scan_dtheta<DV>, dim3(nmz + p.S * p.G), dim3(256), 0, st, p, nmz);
}

hipError_t launch_scan_dtheta(const KParams& p, hipStream_t st)
{
    switch (p.dv) {
    case 8: launch_sd<8>(p, st); break;
    case 16: launch_sd<16>(p, st); break;
    case 32: launch_sd<32>(p, st); break;
    case 64: launch_sd<64>(p, st); break;
    case 128: launch_sd<128>(p, st); break;
    case 256: launch_sd<256>(p, st); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace swl
