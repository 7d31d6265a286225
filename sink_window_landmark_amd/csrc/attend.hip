// Attention of a call: sinks + ring window on fp16 matrix cores at fp32
// accuracy (hi/lo splits, below), and the far readout in the same block's
// epilogue.
//
// cortiq-engine 0.8.51 src/gpu_wgpu/o1_batch.rs, o1b_attend.  Row i of a
// sub-chunk attends to the sinks and to the last min(w_g, len0+i+1) keys of
// ring ++ chunk, self included, and, when its far field is not empty, to the
// Nystrom far estimate under the same softmax:
//   f_a = scale <q, k~_a>, u_b = sum_a exp(f_a - f_max) mu[a][b] (>= 0 with
//   rect), c = max(c_near, max_b f_max + M'_b), gain_b = u_b e^{f_max+M'_b-c},
//   D_far = sum_b gain_b P_bi, N_far = sum_b gain_b R_b Theta_b
//   + sum_{j0<=j<=i} cf_j v_evicted(j) with cf_j = sum_b gain_b E_bj,
//   both dropped when D_far is not >= 0; P_bi = R_b Z_b + sum_{j<=i} E_bj
//   is the far mass prefix, so D_far = sum_b gain_b R_b Z_b +
//   sum_{j0<=j<=i} cf_j, which is how it is formed here;
//   out = (N_far + sum p v) / max(D_far + sum p, 1e-30), p = e^{s-c}.
// M', R, the incoming mass Z and fac = exp(mx - M') (far_scan), E against
// the sub-chunk's own max mx (far_score) and Theta before the sub-chunk
// (theta_scan, or the state for a single sub-chunk) are ready before this
// kernel runs.
//
// The near part never depends on the far field, so every sub-chunk of a call
// is computed in one launch: one block per (sub-chunk, KV group, group of up
// to 4 query heads; 2 at d = 256), two waves per head, each wave owning 32
// query rows.  A launch of fewer than 256 such blocks splits each one's key
// tiles over several blocks and merges their softmax states before the far
// readout (AT_PART, AT_MERGE below).
// The block's keys (the sinks, then the band of positions its rows reach)
// stream through LDS in tiles of 32 keys shared by all heads of the group
// (the GQA reuse of the pages' Metal and Dory kernels).
//
// fp32 products on fp16 matrix cores (near part).  Each fp32 operand x is
// split into fp16 halves, x = hi + lo * 2^-sc: hi is x rounded to nearest
// and lo the remainder rounded to nearest, scaled by 2^11 (sc = 11) for q
// and k so that it stays a normal number.  A product is
// hi*hi + (hi*lo + lo*hi) * 2^-sc on v_mfma_f32_32x32x16_f16 with fp32
// accumulation (the hi*lo terms of the scores in an accumulator of their
// own); the dropped lo*lo term and the rounding of lo leave at most
// 3 * 2^-22 of |a*b| per product a*b, at a fifth of the fp32 MFMA's time
// for the three products.  Values split unscaled after a power-of-two scale
// per (pass, group) that brings their largest magnitude into [2^13, 2^14)
// (from the value maxima that k_far_score writes; an absolute floor of
// 2^-24 against that), and the softmax weights are kept in (0, 2^15] with a
// sum of at least 2^8 so that theirs stays far below that.  Range of the split
// operands: |k| and |scale * log2(e) * q| at most 65504 (fp16's largest
// finite value); values of any finite magnitude.
//
// MFMA layout (32x32 tiles; lane l, half hf = l/32, n = l%32;
// kappa(v, hf) = (v/4)*8 + hf*4 + v%4 is the row of accumulator v):
//   S^T = K Q^T     A = key rows from LDS (key n; k-step st covers columns
//                   16 st + 8 hf .. +7 of lane l), B = Q^T halves held in
//                   registers (query n).  Lane l's accumulators are keys
//                   kappa(v, hf) of query n, so each lane owns one query's
//                   softmax state.
//   O^T += V^T P^T  accumulators 8t .. 8t+7 of S^T are the B operand of
//                   k-step t; V^T sits in LDS with one row per value column
//                   and the keys of a tile permuted (bits 2 and 3 of the
//                   key index swapped) so that the eight keys a lane needs
//                   are one 16-byte read.
// Key tiles: k_kv_split writes every key of a pass once as fp16 hi/lo tiles
// (32 positions each, aligned to multiples of 32, sinks first) in the exact
// byte layout attention wants in LDS, with the 16-byte chunks of each row
// XOR-swizzled so that the MFMA operand reads are free of bank conflicts;
// attention then stages a tile with plain global-to-LDS copies
// (global_load_lds_dwordx4), with no arithmetic and no registers.
//   The far epilogue chains more products in the same shapes: landmarks
//   (a or b) or in-chunk rows j take the place of keys, and a C-layout
//   accumulator tile is always directly the B operand of the next product.
//   The landmark scores and the far numerator run on split fp16 (the
//   numerator's operands scaled by powers of two, far_numerator), u and the
//   in-chunk coefficients on v_mfma_f32_32x32x2f32.
// Softmax runs online in base 2 (q is pre-scaled by scale*log2 e).
#include "swl_internal.h"
#include "lanes.h"
#include "stages.h"

namespace swl {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int KT = 32;                   // keys per tile

constexpr float LO_UP = 2048.f;          // 2^11: scale of the lo halves of q and k
constexpr float LO_DOWN = 1.f / 2048.f;
// Softmax weights are 2^(s - m + P_EXP) against a reference m that is only
// raised when a score exceeds it by more than TAU (log2 units), so they stay
// in (0, 2^(P_EXP + TAU)] = (0, 2^15], inside fp16 range, while the running
// sum, which holds the weight 2^P_EXP of the key that set m, stays at least
// 2^8: the fp16 remainders' absolute floor (2^-24) is then far below fp32
// rounding of the result.
constexpr float P_EXP = 8.f;
constexpr float TAU = 7.f;

// Block shape per head width: two waves per head, up to four heads per block
// (two at d = 256, so that each wave may use a whole SIMD's registers:
// Q^T and O^T alone take 256 of them).
template <int D>
struct AtCfg {
    static constexpr int HPB = D > 128 ? 2 : 4;   // heads per block
    static constexpr int THREADS = HPB * 2 * 64;
};

__device__ __forceinline__ floatx16 mfma32(float a, float b, floatx16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx16 mfma16(u32x4 a, u32x4 b, floatx16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                  __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

__device__ __forceinline__ int kap(int v, int hf) { return (v >> 2) * 8 + hf * 4 + (v & 3); }

// 2^x as the bare v_exp_f32 (results below 2^-126 flush to 0, which only
// drops softmax weights far below the running maximum)
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void zero16(floatx16& x)
{
#pragma unroll
    for (int v = 0; v < 16; ++v) x[v] = 0.f;
}

__device__ __forceinline__ float half0(unsigned x)
{
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(x & 0xffffu));
}
__device__ __forceinline__ float half1(unsigned x)
{
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(x >> 16));
}

// (a, b) as an fp16 pair rounded to nearest, a in the low half
__device__ __forceinline__ unsigned pk16n(float a, float b)
{
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(unsigned, h);
}

// hi/lo fp16 pairs of (a, b): a = hi + lo / 2^11 when SCALED, else hi + lo
// (the remainder a - hi is exact in fp32).  Both halves round to nearest:
// the split's relative error is at most 2^-22, a fourth of what rounding
// toward zero leaves, and it is what scores of large magnitude carry into
// the weights.  The empty asm pins a and b as rounded fp32 values: without
// it the compiler may contract a caller's product into one use (the fused
// conversion v_fma_mixlo_f16 of the unrounded product) but not the other,
// and the two roundings of hi then differ by an fp16 ulp now and then.
template <bool SCALED>
struct Split {
    unsigned hi, lo;
    __device__ __forceinline__ Split(float a, float b)
    {
        asm("" : "+v"(a), "+v"(b));
        hi = pk16n(a, b);
        const float ra = a - half0(hi), rb = b - half1(hi);
        lo = SCALED ? pk16n(ra * LO_UP, rb * LO_UP) : pk16n(ra, rb);
    }
};

// hi/lo fp16 pairs of (a, b) with a = hi + lo, the remainders taken by
// v_fma_mix_f32 straight from the packed fp16 halves (one instruction per
// element instead of a conversion and a subtraction; exact, as a - hi is)
struct SplitMix {
    unsigned hi, lo;
    __device__ __forceinline__ SplitMix(float a, float b)
    {
        hi = pk16n(a, b);
        float ra, rb;
        asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(ra) : "v"(hi), "v"(a));
        asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(rb) : "v"(hi), "v"(b));
        lo = pk16n(ra, rb);
    }
};

// Position of key bit 2 and bit 3 swapped: the order of a tile's keys in the
// V^T rows (an involution).
__device__ __forceinline__ int kperm(int k) { return (k & ~12) | ((k >> 1) & 4) | ((k << 1) & 8); }

// One key tile in fp16 halves: K hi [KT][KD], K lo [KT][KD] (lo scaled by
// 2^11), V^T hi [D][KT], V^T lo [D][KT] (keys in kperm order), 128 (KD + D)
// bytes, a whole number of 1 KB wave copies.  Logical 16-byte chunk c of K
// row r sits at chunk kchunk(r, c) and chunk c of V^T row rho at
// vchunk(rho, c): the rows that one read instruction touches then start in
// different banks.
template <int D>
struct KvTile {
    static constexpr int KD = D < 16 ? 16 : D;   // key width padded to whole k-steps
    static constexpr int KH = KT * KD;
    static constexpr int VH = D * KT;
    static constexpr int HALVES = 2 * KH + 2 * VH;
    static constexpr int BYTES = 2 * HALVES;
    static constexpr int CPR = KD / 8;                     // chunks of a K row
    static constexpr int RPB = KD >= 128 ? 1 : 128 / KD;   // K rows per 256 bytes
    static constexpr int CMASK = (CPR < 16 ? CPR : 16) - 1;
};
template <int D>
__device__ __forceinline__ int kchunk(int r, int c) { return c ^ ((r / KvTile<D>::RPB) & KvTile<D>::CMASK); }
__device__ __forceinline__ int vchunk(int rho, int c) { return c ^ ((rho >> 2) & 3); }

// 16 bytes from global memory into LDS at lds_base + 16 * lane (M0 holds the
// wave's LDS base).  Inline assembly, so that the compiler does not order
// later LDS reads of the other tile buffer behind it: the kernel waits for
// these copies itself (s_waitcnt, then a barrier) before a tile is read.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds_base)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// n floats from p (the same p in every lane of the wave) read by 32-bit
// element index through a buffer resource: one VGPR offset per load in place
// of 64-bit address arithmetic.  Word 3 of the resource is the raw 32-bit
// format of gfx9 targets.  Callers keep their indexes inside [0, n).
struct FView {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ FView(const float* p, int n)
    {
        // (readfirstlane returns a signed int: each half goes through
        // unsigned, so that the low half does not sign-extend into the high)
        const uint64_t a = reinterpret_cast<uint64_t>(p);
        const uint64_t lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)a);
        const uint64_t hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
        r = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(hi << 32 | lo), (short)0, n * 4, 0x00020000);
    }
    __device__ __forceinline__ float operator[](int i) const
    {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, 0));
    }
};

// Split fp16 halves of 8 values times 2^ex (the scaling is exact): an A
// operand, or the B operand of k-step q of a C-layout tile x (its values
// 8q .. 8q+7 in this lane).  The remainders come from v_fma_mix (the same
// bits as a conversion and a subtraction, in one instruction), after the
// scaled values are pinned as rounded fp32 numbers as in Split.
__device__ __forceinline__ void split8(const float (&a)[8], int ex, u32x4& hi, u32x4& lo)
{
    unsigned h[4], l[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float x = ldexpf(a[2 * k], ex), y = ldexpf(a[2 * k + 1], ex);
        asm("" : "+v"(x), "+v"(y));
        const SplitMix s(x, y);
        h[k] = s.hi;
        l[k] = s.lo;
    }
    hi = u32x4{h[0], h[1], h[2], h[3]};
    lo = u32x4{l[0], l[1], l[2], l[3]};
}
__device__ __forceinline__ void split_b(const floatx16& x, int q, int ex, u32x4& hi, u32x4& lo)
{
    float a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = x[8 * q + e];
    split8(a, ex, hi, lo);
}

// The far numerator, O^T += Theta^T (g R)^T + V_ev^T cf^T, on fp16 matrix
// cores with three split products per k-step as in the near part.  Every
// operand enters its split times a power of two that puts it in fp16 range
// with its remainder far above fp16's floor: the gains and the in-chunk
// coefficients per query by their largest magnitude, the evicted values by
// the pass's value exponent, Theta per 32-column block by that block's
// largest magnitude (taken from the loaded values).  Each chain accumulates
// on its own and is scaled back (exactly) as it is added to O.  K-step st of
// tile bt = st / 2 takes, in this lane, rows 32 bt + 16 (st % 2) + 4 hf +
// 8 (e / 4) + e % 4 (e = 0..7): the C-layout rows of the lane's values
// 8 (st % 2) .. + 7, so that the gains and coefficients are B operands as
// they stand.  Theta's loads for a block go out as soon as the block before
// it is split (the first block's before the evicted-value chain, whose
// operands come from LDS).
template <int D, int NB, int MT, int LDF>
__device__ __forceinline__ void far_numerator(floatx16 (&O)[NB], const floatx16 (&gn)[MT], const floatx16 (&cf)[2],
                                              const FView& Th, const float (*Vs)[LDF], int vexp, int m, int ln,
                                              int hf, int st_lo, int st_hi)
{
    constexpr int ST = 2 * MT;   // k-steps of the Theta chain; this wave takes st_lo .. st_hi-1 (gn is zero
                                 // on the others)
    auto krow = [&](int st, int e) { return (st >> 1) * 32 + (st & 1) * 16 + 4 * hf + (e >> 2) * 8 + (e & 3); };
    auto mine = [&](int st) { return st >= st_lo && st < st_hi; };
    float th[ST][8];
    auto load = [&](int blk) {
        const int col = min(blk * 32 + ln, D - 1);
#pragma unroll
        for (int st = 0; st < ST; ++st)
#pragma unroll
            for (int e = 0; e < 8; ++e)   // rows >= m: 0 below
                th[st][e] = mine(st) ? Th[min(krow(st, e), m - 1) * D + col] : 0.f;
    };

    float gmax = 0.f, cmax = 0.f;
#pragma unroll
    for (int bt = 0; bt < MT; ++bt)
#pragma unroll
        for (int t = 0; t < 16; ++t) gmax = fmaxf(gmax, fabsf(gn[bt][t]));
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int t = 0; t < 16; ++t) cmax = fmaxf(cmax, fabsf(cf[jt][t]));
    gmax = pair_max<5>(gmax);   // a query's two lane halves
    cmax = pair_max<5>(cmax);
    const int eg = value_exp_of(gmax), ecf = value_exp_of(cmax);

    if (__any(cmax > 0.f)) {
        u32x4 bh[4], bl[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) split_b(cf[st >> 1], st & 1, ecf, bh[st], bl[st]);
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            const int col = min(blk * 32 + ln, D - 1);
            floatx16 acc;
            zero16(acc);
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                float a[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] = Vs[krow(st, e)][col];
                u32x4 ah, al;
                split8(a, vexp, ah, al);
                acc = mfma16(ah, bh[st], acc);
                acc = mfma16(ah, bl[st], acc);
                acc = mfma16(al, bh[st], acc);
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) O[blk][v] += ldexpf(acc[v], -(vexp + ecf));
        }
    }
    if (__any(gmax > 0.f)) {
        load(0);
        u32x4 bh[ST], bl[ST];
#pragma unroll
        for (int st = 0; st < ST; ++st)
            if (mine(st)) split_b(gn[st >> 1], st & 1, eg, bh[st], bl[st]);
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            float tm = 0.f;
#pragma unroll
            for (int st = 0; st < ST; ++st)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (krow(st, e) >= m) th[st][e] = 0.f;
                    tm = fmaxf(tm, fabsf(th[st][e]));
                }
            const int et = __builtin_amdgcn_readfirstlane(value_exp_of(wmax(tm)));
            u32x4 ah[ST], al[ST];
#pragma unroll
            for (int st = 0; st < ST; ++st)
                if (mine(st)) split8(th[st], et, ah[st], al[st]);
            if (blk + 1 < NB) load(blk + 1);
            floatx16 acc;
            zero16(acc);
#pragma unroll
            for (int st = 0; st < ST; ++st)
                if (mine(st)) {
                    acc = mfma16(ah[st], bh[st], acc);
                    acc = mfma16(ah[st], bl[st], acc);
                    acc = mfma16(al[st], bh[st], acc);
                }
#pragma unroll
            for (int v = 0; v < 16; ++v) O[blk][v] += ldexpf(acc[v], -(et + eg));
        }
    }
}

// ---------------------------------------------------------------------------
// k_kv_split: the key tiles of a pass.  One block per (group, tile): tiles
// 0 .. nst-1 hold the sinks, tile nst + j the window positions 32 j ..
// 32 j + 31 (ring positions, then the pass's rows), up to the last position
// of the pass; rows past the end repeat the last real key (attention masks
// them).  Values are split times the pass's power of two (value_exp), which
// attention takes back out of its value sums.
// ---------------------------------------------------------------------------
template <int D>
constexpr int kv_lds_floats() { return 2 * KT * (D + 1); }

template <int D>
__device__ __forceinline__ void kv_split_body(const KParams& p, int64_t bid, float* lds)
{
    using L = KvTile<D>;
    float(*const kf)[D + 1] = reinterpret_cast<float(*)[D + 1]>(lds);   // [KT][D + 1]
    float(*const vf)[D + 1] = reinterpret_cast<float(*)[D + 1]>(lds + KT * (D + 1));
    const int t = (int)(bid % p.kv_tiles), g = (int)(bid / p.kv_tiles);
    const int nst = (p.ns + KT - 1) / KT;
    const GMeta c = load_gmeta(p.meta, g, p.W);
    const int last = c.len0 + p.T - 1;   // last window position of the pass
    if (t >= nst && (t - nst) * KT > last) return;
    const int vexp = value_exp(p, g);   // values enter their split times 2^vexp
    for (int e = threadIdx.x; e < KT * (D / 4); e += 256) {
        const int r = e / (D / 4), c4 = (e % (D / 4)) * 4;
        const float* kp;
        const float* vp;
        const float* kt = nullptr;   // RoPE table row of a key from the pass's rows
        if (t < nst) {
            const int64_t off = ((int64_t)g * p.ns + min(t * KT + r, p.ns - 1)) * D;
            kp = p.sink_k + off;
            vp = p.sink_v + off;
        } else {
            const int pos = min((t - nst) * KT + r, last);
            kp = key_row(p, c, g, pos);
            vp = val_row(p, c, g, pos);
            if (p.rope && pos >= c.len0) kt = p.rope + (int64_t)(pos - c.len0) * D;
        }
        const float4 kx = rope4(kp, kt, c4, D);
        const float4 vx = *reinterpret_cast<const float4*>(vp + c4);
        kf[r][c4] = kx.x; kf[r][c4 + 1] = kx.y; kf[r][c4 + 2] = kx.z; kf[r][c4 + 3] = kx.w;
        vf[r][c4] = vx.x; vf[r][c4 + 1] = vx.y; vf[r][c4 + 2] = vx.z; vf[r][c4 + 3] = vx.w;
    }
    __syncthreads();
    unsigned short* out = p.kvs + ((int64_t)g * p.kv_tiles + t) * L::HALVES;
    // K: row r, logical chunk cc = columns 8 cc .. 8 cc + 7 (zero past D)
    for (int e = threadIdx.x; e < KT * L::CPR; e += 256) {
        const int r = e / L::CPR, cc = e % L::CPR;
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = cc * 8 + j < D ? kf[r][min(cc * 8 + j, D - 1)] : 0.f;
        const Split<true> s0(x[0], x[1]), s1(x[2], x[3]), s2(x[4], x[5]), s3(x[6], x[7]);
        const int dst = r * L::KD + kchunk<D>(r, cc) * 8;
        *reinterpret_cast<u32x4*>(out + dst) = u32x4{s0.hi, s1.hi, s2.hi, s3.hi};
        *reinterpret_cast<u32x4*>(out + L::KH + dst) = u32x4{s0.lo, s1.lo, s2.lo, s3.lo};
    }
    // V^T: value column rho, logical chunk cc = key slots 8 cc .. 8 cc + 7
    unsigned short* vo = out + 2 * L::KH;
    for (int e = threadIdx.x; e < D * 4; e += 256) {
        const int rho = e >> 2, cc = e & 3;
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = ldexpf(vf[kperm(cc * 8 + j)][rho], vexp);
        const Split<false> s0(x[0], x[1]), s1(x[2], x[3]), s2(x[4], x[5]), s3(x[6], x[7]);
        const int dst = rho * KT + vchunk(rho, cc) * 8;
        *reinterpret_cast<u32x4*>(vo + dst) = u32x4{s0.hi, s1.hi, s2.hi, s3.hi};
        *reinterpret_cast<u32x4*>(vo + L::VH + dst) = u32x4{s0.lo, s1.lo, s2.lo, s3.lo};
    }
}

// The key tiles of a pass in one launch with either the far scan (a call
// whose accumulator scan runs in its commit) or the accumulator scan (after
// a far scan launch; with its commit of Theta, M and Z): blocks [0, nmz)
// run the far scan, the next nth the accumulator scan (stages.h), the rest
// split tiles.  None waits on another.
template <int D>
__global__ __launch_bounds__(256) void k_theta_kv(KParams p, int nmz, int nth)
{
    __shared__ __align__(16) float lds[kv_lds_floats<D>()];
    const int b = blockIdx.x;
    if (b < nmz) mz_scan_body(p, b);
    else if (b < nmz + nth) theta_scan_body(p, true, b - nmz);
    else kv_split_body<D>(p, (int64_t)b - nmz - nth, lds);
}

// MODE: AT_FULL, one block per (sub-chunk, group, head group) over all of its
// key tiles; AT_PART, p.nsp blocks per (sub-chunk, group, head group), each
// over one contiguous range of the tiles, writing its softmax state (running
// reference, mass, O^T) to p.apart; AT_MERGE, one block per (sub-chunk,
// group, head), or per half of its query rows, that merges those states and
// runs the far readout.
// The split serves launches with few blocks (a single sub-chunk, short
// prompts), where one block per sub-chunk would leave most CUs idle.
constexpr int AT_FULL = 0, AT_PART = 1, AT_MERGE = 2;
// splits of one work item's key tiles at most (12: at a single max-window
// sub-chunk, more splits shorten the split blocks by more than the merge of
// their records lengthens)
constexpr int AT_MAX_SPLITS = 12;

// Block shape per mode: a merge block has two waves, each on a SIMD of its own,
// so that the few merge blocks of a small call spread their far readouts over
// more CUs.  It takes one head, a wave per half of the query rows, or, in a
// split merge (p.msplit), one half of one head's rows: its waves then share
// the rows and split the landmarks, the first taking the near part and the
// first landmark tile, the second the other tile (the far numerator and mass
// are sums over landmarks), and the two meet in LDS for the far-mass guard
// and the output.  It reads the split blocks' records by their shape (AtCfg).
template <int D, int MODE>
struct AtShape {
    static constexpr int HPB = MODE == AT_MERGE ? 1 : AtCfg<D>::HPB;
    static constexpr int THREADS = HPB * 2 * 64;
};

template <int D, int MT, int MODE>
__global__ __launch_bounds__((AtShape<D, MODE>::THREADS)) void k_attend(KParams p)
{
    constexpr int AT_THREADS = AtShape<D, MODE>::THREADS;
    constexpr int HPB = AtShape<D, MODE>::HPB;
    constexpr int NB = D >= 32 ? D / 32 : 1;  // 32-row blocks of O^T
    using L = KvTile<D>;
    constexpr int KD = L::KD;
    constexpr int NS = KD / 16;               // k-steps of a score tile
    constexpr int BUF = L::HALVES;            // one tile buffer (fp16 halves)
    constexpr int NCH = L::BYTES / 1024;      // 1 KB wave copies of a tile
    constexpr int NW = AT_THREADS / 64;
    constexpr int LDF = D + 4;                // fp32 row stride of the epilogue's tiles
    // key-tile buffers: tile t is read while the copies of tiles t+1 ..
    // t+NBUF-1 are in flight (three where they fit in LDS)
    constexpr int NBUF = D > 128 ? 2 : 3;
    constexpr int NEAR_BYTES = MODE == AT_MERGE ? 0 : NBUF * L::BYTES;   // (merge blocks hold no key tiles)
    constexpr int KTB = 2 * 2 * L::KH * 2;     // landmark keys as two fp16 hi/lo K tiles
    // and, in full blocks where it fits, E of the block's heads (rows padded
    // to 72 floats, so that the two row groups a read touches fall in
    // different banks; merge blocks, whose LDS sets how many share a CU,
    // read E from memory)
    constexpr int ELD = SUB + 8;
    constexpr int FAR_BYTES0 = KTB + 2 * KT * LDF * 4 + HPB * 4 * 64 * 4;
    constexpr int E_BYTES = HPB * 64 * ELD * 4;
    constexpr bool E_LDS = MODE == AT_FULL && FAR_BYTES0 + E_BYTES <= 160 * 1024;
    constexpr int FAR_BYTES = FAR_BYTES0 + (E_LDS ? E_BYTES : 0);
    // a split merge block's two waves exchange their far masses (XD, after
    // the staged tiles) and the second wave's numerator (over the landmark
    // keys' tiles, no longer read by then)
    constexpr int XD_BYTES = MODE == AT_MERGE ? 2 * 32 * 4 : 0;
    static_assert(64 * NB * 16 * 4 <= KTB, "a wave's O^T fits where the landmark keys were staged");
    constexpr int SMEM0 = NEAR_BYTES > FAR_BYTES ? NEAR_BYTES : FAR_BYTES;
    constexpr int SMEM = SMEM0 + XD_BYTES;
    constexpr float LOG2E = 1.4426950408889634f;
    __shared__ __align__(16) unsigned char smem[SMEM];
    unsigned short* const tiles = reinterpret_cast<unsigned short*>(smem);
    // the epilogue reuses the memory: landmark keys (m <= 64 rows) as fp16
    // hi/lo K tiles and the sub-chunk's evicted values (64 rows) in fp32
    unsigned short* const Kt = reinterpret_cast<unsigned short*>(smem);
    float(*const Vs)[LDF] = reinterpret_cast<float(*)[LDF]>(smem + KTB);
    // and the post-sub-chunk max M', rescale R, incoming mass Z and E's
    // factor of each head's landmarks
    float(*const MR)[4][64] = reinterpret_cast<float(*)[4][64]>(smem + KTB + 2 * KT * LDF * 4);
    float(*const ES)[64][ELD] = reinterpret_cast<float(*)[64][ELD]>(smem + FAR_BYTES0);   // [head][b][j]
    float(*const XD)[32] = reinterpret_cast<float(*)[32]>(smem + SMEM0);

    // work item = (sub-chunk, group, head group), dealt to XCDs as ranges of
    // sub-chunks (range_item); a split block also takes split sp of the
    // item's key tiles, a merge block of a split merge query half sp of one
    // head
    const int hgroups = (p.H + HPB - 1) / HPB;
    const bool msplit = MODE == AT_MERGE && MT == 2 && p.msplit;   // (two landmark tiles to split)
    const int nsp = MODE == AT_PART ? p.nsp : msplit ? 2 : 1;
    int s, gi, sp;
    range_item(xcd_work_item(blockIdx.x, p.S * p.G * hgroups * nsp), p.S, p.G * hgroups, nsp, s, gi, sp);
    const int g = gi % p.G, hgrp = gi / p.G;
    const int w = s + p.S * gi;   // the (sub-chunk, group, head group) item
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int hf = lane >> 5, ln = lane & 31;
    const int h = hgrp * HPB + (wave >> 1);
    const bool active = h < p.H;
    const int gh = g * p.H + h;
    const int r0 = s * SUB;
    const int ks = min(SUB, p.T - r0);
    const GMeta c = load_gmeta(p.meta, g, p.W);
    // the key tiles hold the values times 2^vexp: the near value sums carry
    // that factor until the epilogue
    const int vexp = MODE == AT_PART ? 0 : value_exp(p, g);
    const int base = c.len0 + r0;                   // position of chunk row 0
    const int lo_blk = max(0, base - c.wg + 1);
    const int hi_blk = base + ks - 1;
    const int ia = (msplit ? sp : wave & 1) * 32;
    // the landmark tile this wave takes in the far readout: the waves of a
    // split merge block share their rows and split the landmarks between
    // them; other waves take all (-1)
    const int rt = msplit ? wave & 1 : -1;
    auto my_tile = [&](int bt) { return rt < 0 || bt == rt; };
    const int i = ia + ln;                          // this lane's query row
    const int hi_q = base + i;
    const int lo_q = max(0, hi_q - c.wg + 1);
    const bool wave_rows = active && ia < ks;
    const int ib = min(ks, ia + 32) - 1;
    const int w_lo = max(0, base + ia - c.wg + 1);  // lowest position a row of the wave sees
    const int w_hi = base + ib;                      // highest
    const int lo_ib = max(0, base + ib - c.wg + 1);  // every row of the wave sees [lo_ib, base+ia]

    floatx16 O[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) zero16(O[b]);
    float mrun = -INFINITY, lsum = 0.f;

    // split-window partials, one record of PF4 float4 per (item, split,
    // thread): the running reference, the mass, then O^T.  AT_PART stores
    // this lane's state after its tiles; AT_MERGE combines the p.nsp states
    // of its lane against their largest reference, before the query halves
    // take their registers (four records in flight at a time).
    constexpr int PF4 = (NB * 16 + 2 + 3) / 4;
    if constexpr (MODE == AT_MERGE) {
        // this head's records among those of the split blocks' item (their
        // shape: PH heads, PT threads)
        constexpr int PT = AtCfg<D>::THREADS, PH = AtCfg<D>::HPB;
        const int wp = s + p.S * (g + p.G * (h / PH));
        const int tp = (h % PH) * 128 + ia * 2 + lane;   // that block's thread of this lane's query
        const float4* pp = reinterpret_cast<const float4*>(p.apart) + ((int64_t)wp * p.nsp * PT + tp) * PF4;
        // the largest reference first, every record's head in flight at once
        // (splits past nsp read the last record again)
        float xm[AT_MAX_SPLITS];
#pragma unroll
        for (int k = 0; k < AT_MAX_SPLITS; ++k) xm[k] = pp[(int64_t)min(k, p.nsp - 1) * PT * PF4].x;
#pragma unroll
        for (int k = 0; k < AT_MAX_SPLITS; ++k) mrun = fmaxf(mrun, xm[k]);
        // the first wave takes the near part; the second needs the reference alone
#pragma unroll 4
        for (int k = 0; k < (rt <= 0 ? p.nsp : 0); ++k) {
            const float4* pk = pp + (int64_t)k * PT * PF4;
            float4 r[PF4];
#pragma unroll
            for (int f = 0; f < PF4; ++f) r[f] = pk[f];
            const float* x = reinterpret_cast<const float*>(r);
            const float wk = x[0] == -INFINITY ? 0.f : ex2(x[0] - mrun);   // a split that saw no key adds nothing
            lsum += wk * x[1];
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) O[b][v] += wk * x[2 + b * 16 + v];
        }
    }

    // Q^T halves of this lane: q[r0+i][gh][16 st + 8 hf + e] * scale * log2 e
    u32x4 qh[NS], ql[NS];
    {
        const float qs = p.scale * LOG2E;
        const bool ok = active && i < ks;
        const float* qr = p.q + ((int64_t)(r0 + i) * p.nh + gh) * D;
        const float* qt = p.rope ? p.rope + (int64_t)(r0 + i) * D : nullptr;   // RoPE on the way in
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const int d0 = st * 16 + hf * 8;
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x;
            if (ok & (d0 < D)) {
                x = rope4(qr, qt, d0, D);
                y = rope4(qr, qt, d0 + 4, D);
            }
            const Split<true> s0(x.x * qs, x.y * qs), s1(x.z * qs, x.w * qs);
            const Split<true> s2(y.x * qs, y.y * qs), s3(y.z * qs, y.w * qs);
            qh[st] = u32x4{s0.hi, s1.hi, s2.hi, s3.hi};
            ql[st] = u32x4{s0.lo, s1.lo, s2.lo, s3.lo};
        }
    }

    // tiles: the sinks, then the aligned window tiles j0 .. j1 that meet the
    // block's positions lo_blk .. hi_blk
    const int nst = (p.ns + KT - 1) / KT;
    const int j0 = lo_blk / KT;
    const int ntiles = nst + hi_blk / KT - j0 + 1;
    const unsigned short* kvg = p.kvs + (int64_t)g * p.kv_tiles * BUF + lane * 8;
    auto issue = [&](int tt, int buf) {
        const unsigned short* src = kvg + (int64_t)(tt < nst ? tt : tt + j0) * BUF;
#pragma unroll
        for (int ch = wave; ch < NCH; ch += NW)
            dma16(src + ch * 512, __builtin_amdgcn_readfirstlane(lds_addr(tiles + buf * BUF + ch * 512)));
    };

    // ---- near part: online softmax over the key tiles ----
    // the block's tiles: all of them, split sp's range of them, or none (merge)
    const int per = (ntiles + nsp - 1) / nsp;
    const int tA = MODE == AT_MERGE ? 0 : min(ntiles, sp * per);
    const int tB = MODE == AT_MERGE ? 0 : min(ntiles, tA + per);
    // a wave's copies per tile, when every wave makes as many (the count it
    // may leave in flight while waiting for an earlier tile; else it waits
    // for all)
    constexpr int KPW = NCH % NW == 0 ? NCH / NW : 0;
    constexpr int LEFT = (NBUF - 2) * KPW;   // copies of the tiles after the next one
    for (int t = 0; t < NBUF - 1; ++t)
        if (tA + t < tB) issue(tA + t, t);
    int buf = 0;
#pragma unroll 1
    for (int tt = tA; tt < tB; ++tt, buf = buf + 1 == NBUF ? 0 : buf + 1) {
        // this wave's copies of tile tt have landed (those of later tiles may
        // still be in flight: vmcnt counts only the tile copies here)
        if (LEFT > 0 && tt + NBUF - 2 < tB)
            __builtin_amdgcn_s_waitcnt((LEFT & 15) | (7 << 4) | (15 << 8) | (((LEFT >> 4) & 3) << 14));
        else
            __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();   // ... and every wave's; tile tt-1 is no longer read
        if (tt + NBUF - 1 < tB) {
            const int nb = buf + NBUF - 1 < NBUF ? buf + NBUF - 1 : buf - 1;   // the buffer of tile tt-1
            issue(tt + NBUF - 1, nb);
        }

        const bool sink = tt < nst;
        const int tb = sink ? tt * KT : (j0 + tt - nst) * KT;
        const bool relevant = wave_rows && (sink || (tb <= w_hi && tb + KT - 1 >= w_lo));
        if (!relevant) continue;

        // the score accumulator starts at -bias, the offset of this tile's
        // weights against the reference as it stands, so the scores come out
        // biased and the weights need no subtraction of their own (a tile
        // that raises the reference shifts them once more, below)
        const float bias = (mrun == -INFINITY ? 0.f : mrun) - P_EXP;
        floatx16 sh, sx;
#pragma unroll
        for (int v = 0; v < 16; ++v) sh[v] = -bias;
        zero16(sx);
        const unsigned short* kr = tiles + buf * BUF + ln * KD;
        // a wave in an MFMA stretch gets issue priority over its SIMD partner
        // in its softmax stretch, so the two overlap; in the score stretch
        // waves 0-3 also rank above waves 4-7, so that waves sharing a SIMD
        // tend to drift apart instead of reaching their softmax stretches
        // together
        if (wave < 4) __builtin_amdgcn_s_setprio(2);
        else __builtin_amdgcn_s_setprio(1);
        // (the operands of step st+1 are read before the products of step st
        // are issued, so the LDS latency hides behind them)
        u32x4 ah = *reinterpret_cast<const u32x4*>(kr + kchunk<D>(ln, hf) * 8);
        u32x4 al = *reinterpret_cast<const u32x4*>(kr + L::KH + kchunk<D>(ln, hf) * 8);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            u32x4 ahn = ah, aln = al;
            if (st + 1 < NS) {
                const int ck = kchunk<D>(ln, 2 * st + 2 + hf) * 8;
                ahn = *reinterpret_cast<const u32x4*>(kr + ck);
                aln = *reinterpret_cast<const u32x4*>(kr + L::KH + ck);
            }
            sh = mfma16(ah, qh[st], sh);
            sx = mfma16(ah, ql[st], sx);
            sx = mfma16(al, qh[st], sx);
            ah = ahn;
            al = aln;
        }
        // issue order: the first two steps' reads, then per step its three
        // products and the reads of the step after next
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
            if (st + 2 < NS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        // the value product's first operands are read now, so that their LDS
        // latency hides behind the softmax
        const unsigned short* vr = tiles + buf * BUF + 2 * L::KH;
        auto vaddr = [&](int k) {
            const int rho = min((k >> 1) * 32 + ln, D - 1);
            return rho * KT + vchunk(rho, 2 * (k & 1) + hf) * 8;
        };
        u32x4 vh = *reinterpret_cast<const u32x4*>(vr + vaddr(0));
        u32x4 vl = *reinterpret_cast<const u32x4*>(vr + L::VH + vaddr(0));
        floatx16 sacc;
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[v] = fmaf(sx[v], LO_DOWN, sh[v]);
        // sinks are always visible; the window key at position tb + kappa is
        // visible to row i when lo_q <= pos <= hi_q (every row of the wave
        // sees every key of a "full" tile)
        float tmax = -INFINITY;
        // (the tile test is uniform over the wave: a scalar branch)
        const int full_tile = __builtin_amdgcn_readfirstlane((int)(!sink && tb >= lo_ib && tb + KT - 1 <= base + ia));
        if (full_tile) {
#pragma unroll
            for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, sacc[v]);
        } else if (sink) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float sv = tb + kap(v, hf) < p.ns ? sacc[v] : -INFINITY;
                sacc[v] = sv;
                tmax = fmaxf(tmax, sv);
            }
        } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int pos = tb + kap(v, hf);
                const float sv = (pos >= lo_q && pos <= hi_q) ? sacc[v] : -INFINITY;
                sacc[v] = sv;
                tmax = fmaxf(tmax, sv);
            }
        }
        tmax = pair_max<5>(tmax);   // with the lane 32 away (permlane swap, no LDS)
        // raise the reference (and rescale the running sums) only when some
        // query's score exceeds it by more than TAU
        // (tmax is biased: the score maximum is tmax + bias)
        if (__any(tmax + bias > mrun + TAU)) {
            const float mnew = fmaxf(mrun, tmax + bias);
            const float alpha = mnew == -INFINITY ? 1.f : ex2(mrun - mnew);
            lsum *= alpha;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) O[b][v] *= alpha;
            mrun = mnew;
            // to the raised reference (a lane still without one keeps its bias)
            const float shift = ((mrun == -INFINITY ? 0.f : mrun) - P_EXP) - bias;
#pragma unroll
            for (int v = 0; v < 16; ++v) sacc[v] -= shift;
        }
        float ts = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float pv = ex2(sacc[v]);
            sacc[v] = pv;
            ts += pv;
        }
        lsum += ts;
        u32x4 ph[2], pl[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const SplitMix s0(sacc[8 * t], sacc[8 * t + 1]), s1(sacc[8 * t + 2], sacc[8 * t + 3]);
            const SplitMix s2(sacc[8 * t + 4], sacc[8 * t + 5]), s3(sacc[8 * t + 6], sacc[8 * t + 7]);
            ph[t] = u32x4{s0.hi, s1.hi, s2.hi, s3.hi};
            pl[t] = u32x4{s0.lo, s1.lo, s2.lo, s3.lo};
        }
        __builtin_amdgcn_s_setprio(1);
        // step (blk, t) = step k = 2 blk + t; operands of step k+1 are read
        // before the products of step k, and the products of a step go to one
        // accumulator while the next step's go to another
#pragma unroll
        for (int k = 0; k < 2 * NB; ++k) {
            u32x4 vhn = vh, vln = vl;
            if (k + 1 < 2 * NB) {
                vhn = *reinterpret_cast<const u32x4*>(vr + vaddr(k + 1));
                vln = *reinterpret_cast<const u32x4*>(vr + L::VH + vaddr(k + 1));
            }
            const int blk = k >> 1, t = k & 1;
            O[blk] = mfma16(vh, ph[t], O[blk]);
            O[blk] = mfma16(vh, pl[t], O[blk]);
            O[blk] = mfma16(vl, ph[t], O[blk]);
            vh = vhn;
            vl = vln;
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int k = 0; k < 2 * NB; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
            if (k + 2 < 2 * NB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_s_setprio(0);
    }
    if constexpr (MODE == AT_PART) {
        float4 r[PF4];
        float* x = reinterpret_cast<float*>(r);
        x[0] = mrun;
        x[1] = lsum;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) x[2 + b * 16 + v] = O[b][v];
#pragma unroll
        for (int f = NB * 16 + 2; f < PF4 * 4; ++f) x[f] = 0.f;
        float4* pp = reinterpret_cast<float4*>(p.apart) + (((int64_t)w * nsp + sp) * AT_THREADS + tid) * PF4;
#pragma unroll
        for (int f = 0; f < PF4; ++f) pp[f] = r[f];
        return;
    }
    float den = pair_sum<5>(lsum);   // near mass relative to mrun

    // ---- far readout (o1b_attend's far half) ----
    const SubMeta sm = sub_meta(c, r0);
    const int jlo = max(sm.j0, 0);
    const bool blk_far = sm.nfar0 > 0 || jlo < ks;   // some row of the block has far terms
    if (blk_far) {
        const int m = p.m;
        __syncthreads();  // every wave is done with the key tiles
        // landmark keys of the group -> Ks rows 0..m-1 (zero above m);
        // evicted values of the sub-chunk -> Vs rows 0..63 (zero where none)
        // each kind's loads all go out before its stores (a compile-time
        // count per thread): a few memory round trips, not one per element
        {
            constexpr int NE = 2 * KT * (D / 4), NU = (NE + AT_THREADS - 1) / AT_THREADS;
            float4 vx[NU];
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int e = tid + u * AT_THREADS;
                const int row = min(e / (D / 4), 2 * KT - 1), c4 = (e % (D / 4)) * 4;
                const int rr = min(max(row, jlo), ks - 1);   // a row that evicts (loads take no lane condition)
                vx[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (jlo < ks) vx[u] = *reinterpret_cast<const float4*>(val_row(p, c, g, c.len0 + r0 + rr - c.wg) + c4);
            }
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int e = tid + u * AT_THREADS;
                const int row = e / (D / 4), c4 = (e % (D / 4)) * 4;
                const bool ev = row >= jlo && row < ks;
                if (e < NE) *reinterpret_cast<float4*>(&Vs[row][c4]) = ev ? vx[u] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        // landmark row a = 32 at + r of K tile at, columns past D zero
        {
            constexpr int NE = 2 * KT * (KD / 4), NU = (NE + AT_THREADS - 1) / AT_THREADS;
            float4 kx[NU];
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int e = tid + u * AT_THREADS;
                const int row = min(e / (KD / 4), 2 * KT - 1), c4 = (e % (KD / 4)) * 4;
                kx[u] = *reinterpret_cast<const float4*>(p.k_tilde + ((int64_t)g * m + min(row, m - 1)) * D + min(c4, D - 4));
            }
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int e = tid + u * AT_THREADS;
                const int row = e / (KD / 4), c4 = (e % (KD / 4)) * 4;
                const bool live = (row < m) & (c4 < D);
                const Split<true> s0(live ? kx[u].x : 0.f, live ? kx[u].y : 0.f), s1(live ? kx[u].z : 0.f, live ? kx[u].w : 0.f);
                const int r = row & 31;
                unsigned short* t = Kt + (row >> 5) * 2 * L::KH + r * KD + kchunk<D>(r, c4 >> 3) * 8 + (c4 & 4);
                if (e < NE) {
                    *reinterpret_cast<u32x2*>(t) = u32x2{s0.hi, s1.hi};
                    *reinterpret_cast<u32x2*>(t + L::KH) = u32x2{s0.lo, s1.lo};
                }
            }
        }
        {
            constexpr int NE = HPB * 4 * 64, NU = (NE + AT_THREADS - 1) / AT_THREADS;
            float x[NU];
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int e = min(tid + u * AT_THREADS, NE - 1);
                const int hh = e >> 8, which = (e >> 6) & 3, b = e & 63;
                const int ghh = g * p.H + min(hgrp * HPB + hh, p.H - 1);
                const float* src = which == 0 ? p.Ms : which == 1 ? p.Rs : which == 2 ? p.TZ : p.FAC;
                x[u] = src[((int64_t)s * p.nh + ghh) * m + min(b, m - 1)];
            }
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int e = tid + u * AT_THREADS;
                if (e < NE) MR[e >> 8][(e >> 6) & 3][e & 63] = x[u];
            }
        }
        if constexpr (E_LDS) {
            // E of each head of the block: [b][j] against the sub-chunk's own
            // max, 0 where row j evicts nothing; rows past m zero
            constexpr int NE = HPB * 64 * (SUB / 4), NU = (NE + AT_THREADS - 1) / AT_THREADS;
            float4 ex[NU];
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int e = min(tid + u * AT_THREADS, NE - 1);
                const int hh = e / (64 * (SUB / 4)), b = (e / (SUB / 4)) & 63, j4 = e % (SUB / 4);
                const int ghh = g * p.H + min(hgrp * HPB + hh, p.H - 1);
                const float* src = p.E + (((int64_t)s * p.nh + ghh) * m + min(b, m - 1)) * SUB + j4 * 4;
                ex[u] = *reinterpret_cast<const float4*>(src);
            }
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int e = tid + u * AT_THREADS;
                const int hh = e / (64 * (SUB / 4)), b = (e / (SUB / 4)) & 63, j4 = e % (SUB / 4);
                if (e < NE)
                    *reinterpret_cast<float4*>(&ES[hh][b][j4 * 4]) = b < m ? ex[u] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        __syncthreads();

        const int farl = sm.nfar0 + (i >= sm.j0 ? i - sm.j0 + 1 : 0);
        const bool lane_far = active && i < ks && farl > 0;
        if (wave_rows) {
            const int64_t nhm = (int64_t)p.nh * m;
            const int64_t ghb0 = (int64_t)s * nhm + (int64_t)gh * m;   // (s, gh, b = 0)
            const float* Ms = MR[wave >> 1][0];   // (b < 64: entries past m are not used)
            const float* Rs = MR[wave >> 1][1];
            const float* Zs = MR[wave >> 1][2];
            const float* Fs = MR[wave >> 1][3];
            const float* Eb = p.E + ghb0 * SUB;   // [b][j] exp(l - mx), 0 where row j evicts nothing
            const FView Th(p.theta_prev + (int64_t)s * p.theta_prev_stride + (int64_t)gh * m * D, m * D);

            // f^T = K~ Q^T (log2 units) from the near part's Q^T halves, three
            // split products per k-step; e = exp2(f - fmax)
            floatx16 ef[MT];
#pragma unroll
            for (int at = 0; at < MT; ++at) {
                floatx16 fh, fx;
                zero16(fh);
                zero16(fx);
                const unsigned short* kr = Kt + at * 2 * L::KH + ln * KD;
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    const int ck = kchunk<D>(ln, 2 * st + hf) * 8;
                    const u32x4 ah = *reinterpret_cast<const u32x4*>(kr + ck);
                    const u32x4 al = *reinterpret_cast<const u32x4*>(kr + L::KH + ck);
                    fh = mfma16(ah, qh[st], fh);
                    fx = mfma16(ah, ql[st], fx);
                    fx = mfma16(al, qh[st], fx);
                }
#pragma unroll
                for (int v = 0; v < 16; ++v) ef[at][v] = fmaf(fx[v], LO_DOWN, fh[v]);
            }
            float fmax = -INFINITY;
#pragma unroll
            for (int at = 0; at < MT; ++at)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    if (at * 32 + kap(v, hf) >= m) ef[at][v] = -INFINITY;
                    fmax = fmaxf(fmax, ef[at][v]);
                }
            fmax = pair_max<5>(fmax);
#pragma unroll
            for (int at = 0; at < MT; ++at)
#pragma unroll
                for (int v = 0; v < 16; ++v) ef[at][v] = ex2(ef[at][v] - fmax);

            // u^T = mu^T e^T: A[b][a] = mu[a][b] straight from memory
            const float* mu = p.mu + (int64_t)gh * m * m;
            floatx16 gn[MT];
#pragma unroll
            for (int bt = 0; bt < MT; ++bt) {
                zero16(gn[bt]);
                if (!my_tile(bt)) continue;
                const int b = bt * 32 + ln;
#pragma unroll
                for (int at = 0; at < MT; ++at) {
                    float av[16];
#pragma unroll
                    for (int t = 0; t < 16; ++t) {
                        const int a = at * 32 + kap(t, hf);
                        av[t] = (a < m && b < m) ? mu[(int64_t)a * m + b] : 0.f;
                    }
#pragma unroll
                    for (int t = 0; t < 16; ++t) gn[bt] = mfma32(av[t], ef[at][t], gn[bt]);
                }
            }
            // common exponent (log2 units), gains, far mass
            float mb[MT][16];
            float mmax = -INFINITY;
#pragma unroll
            for (int bt = 0; bt < MT; ++bt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int b = bt * 32 + kap(v, hf);
                    mb[bt][v] = Ms[b] * LOG2E;   // (rows past m hold row m-1: read, then select)
                    if (b >= m) mb[bt][v] = -INFINITY;
                    mmax = fmaxf(mmax, mb[bt][v]);
                }
            mmax = pair_max<5>(mmax);
            const float cexp = lane_far ? fmaxf(mrun, fmax + mmax) : mrun;
            // gains, and the part of the far mass the sub-chunk starts from:
            // sum_b gain_b R_b Z_b (the mass of the rows it evicts is the sum
            // of the in-chunk coefficients below)
            float dfar = 0.f;
#pragma unroll
            for (int bt = 0; bt < MT; ++bt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    if (!my_tile(bt)) continue;
                    const int b = bt * 32 + kap(v, hf);
                    float u = gn[bt][v];
                    if (p.rect) u = fmaxf(u, 0.f);
                    float gain = u * ex2(fmax + mb[bt][v] - cexp);
                    float mass = gain * (Rs[b] * Zs[b]);
                    // computed in every lane, then selected: otherwise the
                    // compiler moves the work under the lane condition, a
                    // branch and an LDS wait per element
                    asm volatile("" : "+v"(gain), "+v"(mass));
                    if (!lane_far || b >= m) gain = mass = 0.f;
                    gn[bt][v] = gain;
                    dfar += mass;
                }
            // in-chunk coefficients cf^T = E^T g^T over rows j0 <= j <= i
            // (E against the post-sub-chunk max is the stored one times fac_b)
            floatx16 cf[2];
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                zero16(cf[jt]);
                const int j = jt * 32 + ln;
#pragma unroll
                for (int bt = 0; bt < MT; ++bt) {
                    if (!my_tile(bt)) continue;
                    float av[16];
#pragma unroll
                    for (int t = 0; t < 16; ++t) {
                        const int b = bt * 32 + kap(t, hf);
                        if constexpr (E_LDS) av[t] = ES[wave >> 1][b][j];   // (rows past m hold zeros)
                        else av[t] = b < m ? Eb[(int64_t)b * SUB + j] : 0.f;
                    }
#pragma unroll
                    for (int t = 0; t < 16; ++t) {
                        const int b = min(bt * 32 + kap(t, hf), 63);
                        cf[jt] = mfma32(av[t], gn[bt][t] * Fs[b], cf[jt]);
                    }
                }
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int jj = jt * 32 + kap(v, hf);
                    if (jj < jlo || jj > i) cf[jt][v] = 0.f;
                    dfar += cf[jt][v];
                }
            }
            dfar = pair_sum<5>(dfar);
            if (msplit) {
                // the far mass over both waves' landmarks (the waves of a
                // split merge block share their query rows, so both are here)
                if (hf == 0) XD[wave][ln] = dfar;
                __syncthreads();
                dfar = XD[0][ln] + XD[1][ln];
            }
            const bool have = lane_far && dfar >= 0.f;
            if (!have) {
                dfar = 0.f;
#pragma unroll
                for (int bt = 0; bt < MT; ++bt) zero16(gn[bt]);
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) zero16(cf[jt]);
            }
            // near part to the common exponent, then the far numerator
            // the near weights carry 2^P_EXP, the value sums also 2^vexp
            const float wn = ex2(mrun - cexp - P_EXP);
            const float wo = ldexpf(wn, -vexp);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) O[b][v] *= wo;
            den = den * wn + dfar;
#pragma unroll
            for (int bt = 0; bt < MT; ++bt)
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const int b = bt * 32 + kap(t, hf);
                    const float rb = Rs[b];
                    gn[bt][t] *= b < m ? rb : 0.f;
                }
            far_numerator<D, NB, MT, LDF>(O, gn, cf, Th, Vs, vexp, m, ln, hf, rt < 0 ? 0 : 2 * rt,
                                          rt < 0 ? 2 * MT : 2 * rt + 2);
        }
        if (msplit) {
            // the second wave's share of the numerator to the first, through
            // the landmark keys' place (both waves have passed the far-mass
            // exchange, so both are done with them)
            float* oc = reinterpret_cast<float*>(smem) + lane;
            if (wave_rows && rt == 1)
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int v = 0; v < 16; ++v) oc[(b * 16 + v) * 64] = O[b][v];
            __syncthreads();
            if (wave_rows && rt == 0)
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int v = 0; v < 16; ++v) O[b][v] += oc[(b * 16 + v) * 64];
        }
    }

    if (active && i < ks && rt <= 0) {
        // without a far part the value sums still carry 2^vexp (with one,
        // the near part was brought to the far part's scale above)
        const float inv = ldexpf(1.f / fmaxf(den, 1e-30f), blk_far ? 0 : -vexp);
        float* orow = p.out + ((int64_t)(r0 + i) * p.nh + gh) * D;
        // the output gate, when on, multiplies each element on its way out
        const float* zr = p.gate ? p.gate + ((int64_t)(r0 + i) * p.nh + gh) * D : nullptr;
        const float* sr = p.gate_scale + (int64_t)gh * D;
        // accumulator row rho of block blk is value column 32 blk + rho; rows
        // kappa(4a .. 4a+3, hf) are the adjacent columns 8a + 4hf .. +3
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
            for (int a = 0; a < (D >= 32 ? 4 : D / 8); ++a) {
                const int col = blk * 32 + 8 * a + 4 * hf;
                float4 o = make_float4(O[blk][4 * a] * inv, O[blk][4 * a + 1] * inv, O[blk][4 * a + 2] * inv,
                                       O[blk][4 * a + 3] * inv);
                if (zr) {
                    const float4 z = *reinterpret_cast<const float4*>(zr + col);
                    const float4 s = *reinterpret_cast<const float4*>(sr + col);
                    o = make_float4(o.x * gate_of(z.x, s.x), o.y * gate_of(z.y, s.y), o.z * gate_of(z.z, s.z),
                                    o.w * gate_of(z.w, s.w));
                }
                *reinterpret_cast<float4*>(orow + col) = o;
            }
    }
}

// Splits of the window per (sub-chunk, group, head group) item: enough for
// about 256 blocks, at most AT_MAX_SPLITS, at least 4 key tiles per split,
// and never more than the partials plane holds (256 pairs).
static int attend_splits(const KParams& p, int items)
{
    const int max_tiles = (p.ns + KT - 1) / KT + (p.W + SUB + KT - 1) / KT + 1;
    int n = min(AT_MAX_SPLITS, 256 / max(items, 1));
    n = min(n, max_tiles / 4);
    return max(n, 1);
}

template <int D, int MT>
static hipError_t launch_dm(const KParams& p0, hipStream_t st)
{
    constexpr int HPB = AtCfg<D>::HPB;
    const int items = p0.S * p0.G * ((p0.H + HPB - 1) / HPB);
    KParams p = p0;
    p.nsp = attend_splits(p, items);
    if (p.nsp == 1) {
        hipLaunchKernelGGL((k_attend<D, MT, AT_FULL>), dim3(items), dim3(AtCfg<D>::THREADS), 0, st, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_attend<D, MT, AT_PART>), dim3(items * p.nsp), dim3(AtCfg<D>::THREADS), 0, st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the merge: one block per (sub-chunk, group, head), or per half of its
    // rows when that still leaves at most one block per CU (a few merge
    // blocks run their far readouts as latency-bound chains, which the split
    // halves; many are bound by throughput, which the split's duplicated
    // staging would cost)
    constexpr int MERGE_THREADS = AtShape<D, AT_MERGE>::THREADS;
    const int heads = p.S * p.G * p.H;
    p.msplit = MT == 2 && 2 * heads <= 256;
    hipLaunchKernelGGL((k_attend<D, MT, AT_MERGE>), dim3(heads * (p.msplit ? 2 : 1)), dim3(MERGE_THREADS), 0, st, p);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const KParams& p, hipStream_t st)
{
    return p.m <= 32 ? launch_dm<D, 1>(p, st) : launch_dm<D, 2>(p, st);
}

size_t attend_part_floats(int d)
{
    const int threads = d > 128 ? AtCfg<256>::THREADS : AtCfg<128>::THREADS;
    const int nb = d >= 32 ? d / 32 : 1;
    return (size_t)256 * threads * 4 * ((nb * 16 + 2 + 3) / 4);
}

int kv_tiles(int ns, int W, int S)
{
    // positions of a pass: at most W ring keys, then S sub-chunks of rows
    return (ns + KT - 1) / KT + (W + S * SUB + KT - 1) / KT;
}

size_t kv_tile_bytes(int d) { return (size_t)128 * ((d < 16 ? 16 : d) + d); }

template <int D>
static hipError_t launch_theta_kv_d(const KParams& p, bool mz, bool theta, bool kv, hipStream_t st)
{
    const int64_t nmz = mz ? far_scan_blocks(p) : 0;
    const int64_t nth = theta ? theta_blocks(p) : 0;
    const int64_t nkv = kv ? (int64_t)p.G * p.kv_tiles : 0;
    hipLaunchKernelGGL(k_theta_kv<D>, dim3((unsigned)(nmz + nth + nkv)), dim3(256), 0, st, p, (int)nmz,
                       (int)nth);
    return hipGetLastError();
}

hipError_t launch_theta_kv(const KParams& p, bool mz, bool theta, bool kv, hipStream_t st)
{
    switch (p.d) {
    case 8: return launch_theta_kv_d<8>(p, mz, theta, kv, st);
    case 16: return launch_theta_kv_d<16>(p, mz, theta, kv, st);
    case 32: return launch_theta_kv_d<32>(p, mz, theta, kv, st);
    case 64: return launch_theta_kv_d<64>(p, mz, theta, kv, st);
    case 128: return launch_theta_kv_d<128>(p, mz, theta, kv, st);
    case 256: return launch_theta_kv_d<256>(p, mz, theta, kv, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attend(const KParams& p, hipStream_t st)
{
    switch (p.d) {
    case 8: return launch_d<8>(p, st);
    case 16: return launch_d<16>(p, st);
    case 32: return launch_d<32>(p, st);
    case 64: return launch_d<64>(p, st);
    case 128: return launch_d<128>(p, st);
    case 256: return launch_d<256>(p, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace swl
