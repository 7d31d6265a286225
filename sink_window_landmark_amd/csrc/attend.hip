// Attention of a call: sinks + ring window on fp32 MFMA, and the far readout
// in the same block's epilogue.
//
// cortiq-engine 0.8.51 src/gpu_wgpu/o1_batch.rs, o1b_attend.  Row i of a
// sub-chunk attends to the sinks and to the last min(w_g, len0+i+1) keys of
// ring ++ chunk, self included, and, when its far field is not empty, to the
// Nystrom far estimate under the same softmax:
//   f_a = scale <q, k~_a>, u_b = sum_a exp(f_a - f_max) mu[a][b] (>= 0 with
//   rect), c = max(c_near, max_b f_max + M'_b), gain_b = u_b e^{f_max+M'_b-c},
//   D_far = sum_b gain_b P_bi, N_far = sum_b gain_b R_b Theta_b
//   + sum_{j0<=j<=i} cf_j v_evicted(j) with cf_j = sum_b gain_b E_bj,
//   both dropped when D_far is not >= 0;
//   out = (N_far + sum p v) / max(D_far + sum p, 1e-30), p = e^{s-c}.
// M', R, E, P (far_scan) and Theta before the sub-chunk (theta_scan, or the
// state for a single sub-chunk) are ready before this kernel runs.
//
// The near part never depends on the far field, so every sub-chunk of a call
// is computed in one launch: one block per (sub-chunk, KV group, group of up
// to 4 query heads; 2 at d = 256), two waves per head, each wave owning 32
// query rows.
// The block's keys (the sinks, then the band of positions its rows reach)
// stream through LDS in tiles of 32 keys shared by all heads of the group
// (the GQA reuse of the pages' Metal and Dory kernels).
//
// MFMA layout (v_mfma_f32_32x32x2f32; lane l, half hf = l/32, n = l%32;
// kappa(v, hf) = (v/4)*8 + hf*4 + v%4):
//   S^T = K Q^T     A = key rows (key n; the two d columns of step st are
//                   hf*D/2 + st), B = Q^T held in registers (query n).  The
//                   16 accumulators of lane l are keys kappa(v, hf) of query
//                   n, so each lane owns one query's softmax state.
//   O^T += V^T P^T  accumulator v of S^T is the B operand of step t = v;
//                   A = V^T with value column NB*n + blk for block blk.
//   The far products reuse the same shapes: landmarks (a or b) or in-chunk
//   rows j take the place of keys, and a C-layout accumulator tile is always
//   directly the B operand of the next product.
// Softmax runs online in base 2 (q is pre-scaled by scale*log2 e).
#include "swl_internal.h"

namespace swl {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int KT = 32;  // keys per tile

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

__device__ __forceinline__ int kap(int v, int hf) { return (v >> 2) * 8 + hf * 4 + (v & 3); }

// 2^x as the bare v_exp_f32 (results below 2^-126 flush to 0, which only
// drops softmax weights far below the running maximum)
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void zero16(floatx16& x)
{
#pragma unroll
    for (int v = 0; v < 16; ++v) x[v] = 0.f;
}

// O^T[blk] += A_row^T B for one MFMA step: `row` points at the value row of
// this lane's k index (value column NB*n + blk is A for block blk).
template <int D, int NB>
__device__ __forceinline__ void pv_step(floatx16 (&O)[NB], const float* row, int ln, float b)
{
    if constexpr (NB == 8) {
        const float4 a = *reinterpret_cast<const float4*>(row + 8 * ln);
        const float4 c = *reinterpret_cast<const float4*>(row + 8 * ln + 4);
        O[0] = mfma32(a.x, b, O[0]);
        O[1] = mfma32(a.y, b, O[1]);
        O[2] = mfma32(a.z, b, O[2]);
        O[3] = mfma32(a.w, b, O[3]);
        O[4] = mfma32(c.x, b, O[4]);
        O[5] = mfma32(c.y, b, O[5]);
        O[6] = mfma32(c.z, b, O[6]);
        O[7] = mfma32(c.w, b, O[7]);
    } else if constexpr (NB == 4) {
        const float4 a = *reinterpret_cast<const float4*>(row + 4 * ln);
        O[0] = mfma32(a.x, b, O[0]);
        O[1] = mfma32(a.y, b, O[1]);
        O[2] = mfma32(a.z, b, O[2]);
        O[3] = mfma32(a.w, b, O[3]);
    } else if constexpr (NB == 2) {
        const float2 a = *reinterpret_cast<const float2*>(row + 2 * ln);
        O[0] = mfma32(a.x, b, O[0]);
        O[1] = mfma32(a.y, b, O[1]);
    } else {
        const float a = ln < D ? row[ln] : 0.f;
        O[0] = mfma32(a, b, O[0]);
    }
}

template <int D, int MT>
__global__ __launch_bounds__(AtCfg<D>::THREADS) void k_attend(KParams p)
{
    constexpr int AT_THREADS = AtCfg<D>::THREADS;
    constexpr int HPB = AtCfg<D>::HPB;
    constexpr int NB = D >= 32 ? D / 32 : 1;  // 32-column output blocks
    constexpr int LD = D + 4;                 // LDS row stride
    constexpr int F4 = KT * D / 4;            // float4 per tile matrix
    constexpr int LPT = (F4 + AT_THREADS - 1) / AT_THREADS;
    constexpr float LOG2E = 1.4426950408889634f;
    // two tile buffers of K and of V; the epilogue reuses Ks for the landmark
    // keys (m <= 64 rows) and Vs for the sub-chunk's evicted values (64 rows)
    __shared__ float Ks[2 * KT][LD];
    __shared__ float Vs[2 * KT][LD];

    // work item = (head group, group, sub-chunk), sub-chunk fastest, dealt
    // to XCDs in contiguous runs
    const int hgroups = (p.H + HPB - 1) / HPB;
    const int w = xcd_work_item(blockIdx.x, p.S * p.G * hgroups);
    const int s = w % p.S, g = (w / p.S) % p.G, hgrp = w / (p.S * p.G);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int hf = lane >> 5, ln = lane & 31;
    const int h = hgrp * HPB + (wave >> 1);
    const bool active = h < p.H;
    const int gh = g * p.H + h;
    const int r0 = s * SUB;
    const int ks = min(SUB, p.T - r0);
    const GMeta c = load_gmeta(p.meta, g, p.W);
    const int base = c.len0 + r0;                   // position of chunk row 0
    const int lo_blk = max(0, base - c.wg + 1);
    const int hi_blk = base + ks - 1;
    const int ia = (wave & 1) * 32;
    const int i = ia + ln;                          // this lane's query row
    const int hi_q = base + i;
    const int lo_q = max(0, hi_q - c.wg + 1);
    const bool wave_rows = active && ia < ks;
    const int ib = min(ks, ia + 32) - 1;
    const int w_lo = max(0, base + ia - c.wg + 1);  // lowest position a row of the wave sees
    const int w_hi = base + ib;                      // highest
    const int lo_ib = max(0, base + ib - c.wg + 1);  // every row of the wave sees [lo_ib, base+ia]

    // Q^T fragment of this lane: q[r0+i][gh][hf*D/2 + st], pre-scaled.
    float qf[D / 2];
    {
        const float qs = p.scale * LOG2E;
        const bool ok = active && i < ks;
        const float* qr = p.q + ((int64_t)(r0 + i) * p.nh + gh) * D + hf * (D / 2);
#pragma unroll
        for (int st = 0; st < D / 2; st += 4) {
            float4 x = ok ? *reinterpret_cast<const float4*>(qr + st) : make_float4(0.f, 0.f, 0.f, 0.f);
            qf[st] = x.x * qs;
            qf[st + 1] = x.y * qs;
            qf[st + 2] = x.z * qs;
            qf[st + 3] = x.w * qs;
        }
    }

    const int nst = (p.ns + KT - 1) / KT;
    const int nwt = (hi_blk - lo_blk + KT) / KT;
    const int ntiles = nst + nwt;

    float4 kreg[LPT], vreg[LPT];
    auto load_tile = [&](int tt) {
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int e = tid + u * AT_THREADS;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (e < F4) {
                const int row = e / (D / 4), c4 = (e % (D / 4)) * 4;
                const float* kb = nullptr;
                const float* vb = nullptr;
                uint32_t off = 0;
                if (tt < nst) {
                    const int x = tt * KT + row;
                    if (x < p.ns) {
                        kb = p.sink_k;
                        vb = p.sink_v;
                        off = (uint32_t)(g * p.ns + x) * D;
                    }
                } else {
                    const int pos = lo_blk + (tt - nst) * KT + row;
                    if (pos <= hi_blk) {
                        if (pos < c.len0) {
                            kb = p.ring_k;
                            vb = p.ring_v;
                            off = (uint32_t)(g * p.W + (uint32_t)(c.head0 + pos) % (uint32_t)c.wg) * D;
                        } else {
                            kb = p.k;
                            vb = p.v;
                            off = (uint32_t)((pos - c.len0) * p.G + g) * D;
                        }
                    }
                }
                if (kb) {
                    kx = *reinterpret_cast<const float4*>(kb + off + c4);
                    vx = *reinterpret_cast<const float4*>(vb + off + c4);
                }
            }
            kreg[u] = kx;
            vreg[u] = vx;
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int e = tid + u * AT_THREADS;
            if (e < F4) {
                const int row = e / (D / 4), c4 = (e % (D / 4)) * 4;
                *reinterpret_cast<float4*>(&Ks[buf * KT + row][c4]) = kreg[u];
                *reinterpret_cast<float4*>(&Vs[buf * KT + row][c4]) = vreg[u];
            }
        }
    };

    floatx16 O[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) zero16(O[b]);
    float mrun = -INFINITY, lsum = 0.f;

    // ---- near part: online softmax over the key tiles ----
    load_tile(0);
    for (int tt = 0; tt < ntiles; ++tt) {
        const int buf = tt & 1;
        store_tile(buf);
        __syncthreads();
        if (tt + 1 < ntiles) load_tile(tt + 1);

        const bool sink = tt < nst;
        const int tb = sink ? tt * KT : lo_blk + (tt - nst) * KT;
        const bool relevant = wave_rows && (sink || (tb <= w_hi && tb + KT - 1 >= w_lo));
        if (!relevant) continue;

        floatx16 sacc;
        zero16(sacc);
        const float* kr = &Ks[buf * KT + ln][hf * (D / 2)];
        // a wave in an MFMA stretch gets issue priority over its SIMD partner
        // in its softmax stretch, so the two overlap; in the score stretch
        // waves 0-3 also rank above waves 4-7, so that waves sharing a SIMD
        // tend to drift apart instead of reaching their softmax stretches
        // together
        if (wave < 4) __builtin_amdgcn_s_setprio(2);
        else __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < D / 2; st += 4) {
            const float4 a = *reinterpret_cast<const float4*>(kr + st);
            sacc = mfma32(a.x, qf[st], sacc);
            sacc = mfma32(a.y, qf[st + 1], sacc);
            sacc = mfma32(a.z, qf[st + 2], sacc);
            sacc = mfma32(a.w, qf[st + 3], sacc);
        }
        __builtin_amdgcn_s_setprio(0);
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
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        // rescale the running sums only when some query's maximum rises
        if (__any(tmax > mrun)) {
            const float mnew = fmaxf(mrun, tmax);
            const float alpha = mnew == -INFINITY ? 1.f : ex2(mrun - mnew);
            lsum *= alpha;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) O[b][v] *= alpha;
            mrun = mnew;
        }
        const float msub = mrun == -INFINITY ? 0.f : mrun;
        float ts = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float pv = ex2(sacc[v] - msub);
            sacc[v] = pv;
            ts += pv;
        }
        lsum += ts;
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < 16; ++t) pv_step<D, NB>(O, &Vs[buf * KT + kap(t, hf)][0], ln, sacc[t]);
        __builtin_amdgcn_s_setprio(0);
    }
    float den = lsum + __shfl_xor(lsum, 32, 64);   // near mass relative to mrun

    // ---- far readout (o1b_attend's far half) ----
    const SubMeta sm = sub_meta(c, r0);
    const int jlo = max(sm.j0, 0);
    const bool blk_far = sm.nfar0 > 0 || jlo < ks;   // some row of the block has far terms
    if (blk_far) {
        const int m = p.m;
        __syncthreads();  // every wave is done with the key tiles
        // landmark keys of the group -> Ks rows 0..m-1 (zero above m);
        // evicted values of the sub-chunk -> Vs rows 0..63 (zero where none)
        for (int e = tid; e < 2 * KT * (D / 4); e += AT_THREADS) {
            const int row = e / (D / 4), c4 = (e % (D / 4)) * 4;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (row < m)
                kx = *reinterpret_cast<const float4*>(p.k_tilde + ((int64_t)g * m + row) * D + c4);
            if (row >= jlo && row < ks)
                vx = *reinterpret_cast<const float4*>(val_row(p, c, g, c.len0 + r0 + row - c.wg) + c4);
            *reinterpret_cast<float4*>(&Ks[row][c4]) = kx;
            *reinterpret_cast<float4*>(&Vs[row][c4]) = vx;
        }
        __syncthreads();

        const int farl = sm.nfar0 + (i >= sm.j0 ? i - sm.j0 + 1 : 0);
        const bool lane_far = active && i < ks && farl > 0;
        if (wave_rows) {
            const int64_t nhm = (int64_t)p.nh * m;
            const int64_t ghb0 = (int64_t)s * nhm + (int64_t)gh * m;   // (s, gh, b = 0)
            const float* Ms = p.Ms + ghb0;
            const float* Rs = p.Rs + ghb0;
            const float* Eb = p.E + ghb0 * SUB;                         // [b][j]
            const float* Pb = p.P + ghb0 * SUB;                         // [b][i]
            const float* Th = p.theta_prev + (int64_t)s * p.theta_prev_stride + (int64_t)gh * m * D;

            // f^T = K~ Q^T (log2 units), e = exp2(f - fmax)
            floatx16 ef[MT];
#pragma unroll
            for (int at = 0; at < MT; ++at) {
                zero16(ef[at]);
                const float* kr = &Ks[at * 32 + ln][hf * (D / 2)];
#pragma unroll
                for (int st = 0; st < D / 2; st += 4) {
                    const float4 a = *reinterpret_cast<const float4*>(kr + st);
                    ef[at] = mfma32(a.x, qf[st], ef[at]);
                    ef[at] = mfma32(a.y, qf[st + 1], ef[at]);
                    ef[at] = mfma32(a.z, qf[st + 2], ef[at]);
                    ef[at] = mfma32(a.w, qf[st + 3], ef[at]);
                }
            }
            float fmax = -INFINITY;
#pragma unroll
            for (int at = 0; at < MT; ++at)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    if (at * 32 + kap(v, hf) >= m) ef[at][v] = -INFINITY;
                    fmax = fmaxf(fmax, ef[at][v]);
                }
            fmax = fmaxf(fmax, __shfl_xor(fmax, 32, 64));
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
                    mb[bt][v] = b < m ? Ms[b] * LOG2E : -INFINITY;
                    mmax = fmaxf(mmax, mb[bt][v]);
                }
            mmax = fmaxf(mmax, __shfl_xor(mmax, 32, 64));
            const float cexp = lane_far ? fmaxf(mrun, fmax + mmax) : mrun;
            float dfar = 0.f;
#pragma unroll
            for (int bt = 0; bt < MT; ++bt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int b = bt * 32 + kap(v, hf);
                    float u = gn[bt][v];
                    if (p.rect) u = fmaxf(u, 0.f);
                    const float gain = (lane_far && b < m) ? u * ex2(fmax + mb[bt][v] - cexp) : 0.f;
                    gn[bt][v] = gain;
                    if (b < m && lane_far) dfar += gain * Pb[(int64_t)b * SUB + i];
                }
            dfar += __shfl_xor(dfar, 32, 64);
            const bool have = lane_far && dfar >= 0.f;
            if (!have) {
                dfar = 0.f;
#pragma unroll
                for (int bt = 0; bt < MT; ++bt) zero16(gn[bt]);
            }
            // in-chunk coefficients cf^T = E^T g^T over rows j0 <= j <= i
            floatx16 cf[2];
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                zero16(cf[jt]);
                const int j = jt * 32 + ln;
#pragma unroll
                for (int bt = 0; bt < MT; ++bt) {
                    float av[16];
#pragma unroll
                    for (int t = 0; t < 16; ++t) {
                        const int b = bt * 32 + kap(t, hf);
                        av[t] = b < m ? Eb[(int64_t)b * SUB + j] : 0.f;
                    }
#pragma unroll
                    for (int t = 0; t < 16; ++t) cf[jt] = mfma32(av[t], gn[bt][t], cf[jt]);
                }
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int jj = jt * 32 + kap(v, hf);
                    if (jj < jlo || jj > i) cf[jt][v] = 0.f;
                }
            }
            // near part to the common exponent, then the far numerator
            const float wn = ex2(mrun - cexp);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) O[b][v] *= wn;
            den = den * wn + dfar;
#pragma unroll
            for (int bt = 0; bt < MT; ++bt) {
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const int b = bt * 32 + kap(t, hf);
                    const float r = b < m ? Rs[b] : 0.f;
                    gn[bt][t] *= r;
                }
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const int b = min(bt * 32 + kap(t, hf), m - 1);   // gn is 0 for b >= m
                    pv_step<D, NB>(O, Th + (int64_t)b * D, ln, gn[bt][t]);
                }
            }
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                for (int t = 0; t < 16; ++t) pv_step<D, NB>(O, &Vs[jt * 32 + kap(t, hf)][0], ln, cf[jt][t]);
        }
    }

    if (active && i < ks) {
        const float inv = 1.f / fmaxf(den, 1e-30f);
        float* orow = p.out + ((int64_t)(r0 + i) * p.nh + gh) * D;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int ii = kap(v, hf);
            if constexpr (NB == 8) {
                *reinterpret_cast<float4*>(orow + 8 * ii) =
                    make_float4(O[0][v] * inv, O[1][v] * inv, O[2][v] * inv, O[3][v] * inv);
                *reinterpret_cast<float4*>(orow + 8 * ii + 4) =
                    make_float4(O[4][v] * inv, O[5][v] * inv, O[6][v] * inv, O[7][v] * inv);
            } else if constexpr (NB == 4) {
                *reinterpret_cast<float4*>(orow + 4 * ii) =
                    make_float4(O[0][v] * inv, O[1][v] * inv, O[2][v] * inv, O[3][v] * inv);
            } else if constexpr (NB == 2) {
                *reinterpret_cast<float2*>(orow + 2 * ii) = make_float2(O[0][v] * inv, O[1][v] * inv);
            } else {
                if (ii < D) orow[ii] = O[0][v] * inv;
            }
        }
    }
}

template <int D>
static hipError_t launch_d(const KParams& p, hipStream_t st)
{
    constexpr int HPB = AtCfg<D>::HPB;
    dim3 grid(p.S * p.G * ((p.H + HPB - 1) / HPB));
    if (p.m <= 32) hipLaunchKernelGGL((k_attend<D, 1>), grid, dim3(AtCfg<D>::THREADS), 0, st, p);
    else hipLaunchKernelGGL((k_attend<D, 2>), grid, dim3(AtCfg<D>::THREADS), 0, st, p);
    return hipGetLastError();
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
