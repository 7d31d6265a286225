// Near attention of a call: sinks plus each row's ring window, on fp32 MFMA.
//
// cortiq-engine 0.8.51 src/gpu_wgpu/o1_batch.rs, o1b_attend: row i of a
// sub-chunk attends to the sinks and to the last min(w_g, len0+i+1) keys of
// ring ++ chunk, self included.  That part never depends on the far field,
// so every sub-chunk of a call is computed in one launch: one block per
// (sub-chunk, KV group, group of up to 4 query heads), two waves per head,
// each wave owning 32 query rows.  The block's keys (the sinks, then the band
// of positions its 64 rows reach) stream through LDS in tiles of 32 keys,
// shared by all heads of the group (the GQA reuse the pages' Metal and Dory
// kernels aim for).
//
// MFMA layout (v_mfma_f32_32x32x2f32; lane l, half hf = l/32, n = l%32):
//   S^T = K Q^T    A = K tile rows (key n, two d columns per step, one per
//                  half), B = Q^T (query n) held in registers; the 16
//                  accumulators of lane l are keys (v/4)*8 + hf*4 + v%4 of
//                  query n, so each lane owns one query's softmax state.
//   O^T += V^T P^T the accumulators of S^T are directly the B operand of
//                  step t (keys (t/4)*8 + hf*4 + t%4), A = V^T with value
//                  column NB*n + blk for output block blk.
// Softmax is online, in base 2 (q is pre-scaled by scale*log2(e)).  The
// block writes the normalised near output to `out` and the near max and
// mass of each row to NS; the far readout rescales and merges them.
#include "swl_internal.h"

namespace swl {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int NEAR_THREADS = 512;
constexpr int KT = 32;  // keys per tile

__device__ __forceinline__ floatx16 mfma32(float a, float b, floatx16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(NEAR_THREADS) void k_near(KParams p)
{
    constexpr int NB = D >= 32 ? D / 32 : 1;  // 32-column output blocks
    constexpr int LD = D + 4;                 // LDS row stride
    constexpr int F4 = KT * D / 4;            // float4 per tile matrix
    constexpr int LPT = (F4 + NEAR_THREADS - 1) / NEAR_THREADS;
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr float LN2 = 0.6931471805599453f;
    __shared__ float Ks[2][KT][LD];
    __shared__ float Vs[2][KT][LD];

    const int s = blockIdx.x, g = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int hf = lane >> 5, ln = lane & 31;
    const int h = blockIdx.z * 4 + (wave >> 1);
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
            const int e = tid + u * NEAR_THREADS;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (e < F4) {
                const int row = e / (D / 4), c4 = (e % (D / 4)) * 4;
                const float* kp = nullptr;
                const float* vp = nullptr;
                if (tt < nst) {
                    const int x = tt * KT + row;
                    if (x < p.ns) {
                        kp = p.sink_k + ((int64_t)g * p.ns + x) * D;
                        vp = p.sink_v + ((int64_t)g * p.ns + x) * D;
                    }
                } else {
                    const int pos = lo_blk + (tt - nst) * KT + row;
                    if (pos <= hi_blk) {
                        kp = key_row(p, c, g, pos);
                        vp = val_row(p, c, g, pos);
                    }
                }
                if (kp) {
                    kx = *reinterpret_cast<const float4*>(kp + c4);
                    vx = *reinterpret_cast<const float4*>(vp + c4);
                }
            }
            kreg[u] = kx;
            vreg[u] = vx;
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int e = tid + u * NEAR_THREADS;
            if (e < F4) {
                const int row = e / (D / 4), c4 = (e % (D / 4)) * 4;
                *reinterpret_cast<float4*>(&Ks[buf][row][c4]) = kreg[u];
                *reinterpret_cast<float4*>(&Vs[buf][row][c4]) = vreg[u];
            }
        }
    };

    floatx16 O[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) O[b][v] = 0.f;
    float mrun = -INFINITY, lsum = 0.f;

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

        // S^T tile: 32 keys x 32 queries.
        floatx16 sacc;
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
        const float* kr = &Ks[buf][ln][hf * (D / 2)];
#pragma unroll
        for (int st = 0; st < D / 2; st += 4) {
            const float4 a = *reinterpret_cast<const float4*>(kr + st);
            sacc = mfma32(a.x, qf[st], sacc);
            sacc = mfma32(a.y, qf[st + 1], sacc);
            sacc = mfma32(a.z, qf[st + 2], sacc);
            sacc = mfma32(a.w, qf[st + 3], sacc);
        }
        // masks: sinks always visible; window key at position tb+kappa is
        // visible to row i when lo_q <= pos <= hi_q.
        const bool full = !sink && tb >= lo_ib && tb + KT - 1 <= base + ia;
        float tmax = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int kap = (v >> 2) * 8 + hf * 4 + (v & 3);
            bool ok;
            if (sink) ok = tb + kap < p.ns;
            else if (full) ok = true;
            else {
                const int pos = tb + kap;
                ok = pos >= lo_q && pos <= hi_q;
            }
            const float sv = ok ? sacc[v] : -INFINITY;
            sacc[v] = sv;
            tmax = fmaxf(tmax, sv);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float mnew = fmaxf(mrun, tmax);
        float alpha = 1.f, msub = 0.f;
        if (mnew != -INFINITY) {
            alpha = exp2f(mrun - mnew);
            msub = mnew;
        }
        float ts = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float pv = exp2f(sacc[v] - msub);
            sacc[v] = pv;
            ts += pv;
        }
        lsum = lsum * alpha + ts;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) O[b][v] *= alpha;
        mrun = mnew;
        // O^T += V^T P^T
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int kap = (t >> 2) * 8 + hf * 4 + (t & 3);
            const float* vr = &Vs[buf][kap][0];
            if constexpr (NB == 4) {
                const float4 a = *reinterpret_cast<const float4*>(vr + 4 * ln);
                O[0] = mfma32(a.x, sacc[t], O[0]);
                O[1] = mfma32(a.y, sacc[t], O[1]);
                O[2] = mfma32(a.z, sacc[t], O[2]);
                O[3] = mfma32(a.w, sacc[t], O[3]);
            } else if constexpr (NB == 2) {
                const float2 a = *reinterpret_cast<const float2*>(vr + 2 * ln);
                O[0] = mfma32(a.x, sacc[t], O[0]);
                O[1] = mfma32(a.y, sacc[t], O[1]);
            } else {
                const float a = ln < D ? vr[ln] : 0.f;
                O[0] = mfma32(a, sacc[t], O[0]);
            }
        }
    }

    const float ltot = lsum + __shfl_xor(lsum, 32, 64);
    if (active && i < ks) {
        const float inv = 1.f / ltot;
        float* orow = p.out + ((int64_t)(r0 + i) * p.nh + gh) * D;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int ii = (v >> 2) * 8 + hf * 4 + (v & 3);
            if constexpr (NB == 4) {
                *reinterpret_cast<float4*>(orow + 4 * ii) =
                    make_float4(O[0][v] * inv, O[1][v] * inv, O[2][v] * inv, O[3][v] * inv);
            } else if constexpr (NB == 2) {
                *reinterpret_cast<float2*>(orow + 2 * ii) = make_float2(O[0][v] * inv, O[1][v] * inv);
            } else {
                if (ii < D) orow[ii] = O[0][v] * inv;
            }
        }
        if (hf == 0) {
            float* ns = p.NS + ((int64_t)(r0 + i) * p.nh + gh) * 2;
            ns[0] = mrun * LN2;
            ns[1] = ltot;
        }
    }
}

hipError_t launch_near(const KParams& p, hipStream_t st)
{
    dim3 grid(p.S, p.G, (p.H + 3) / 4);
    switch (p.d) {
    case 8: hipLaunchKernelGGL(k_near<8>, grid, dim3(NEAR_THREADS), 0, st, p); break;
    case 16: hipLaunchKernelGGL(k_near<16>, grid, dim3(NEAR_THREADS), 0, st, p); break;
    case 32: hipLaunchKernelGGL(k_near<32>, grid, dim3(NEAR_THREADS), 0, st, p); break;
    case 64: hipLaunchKernelGGL(k_near<64>, grid, dim3(NEAR_THREADS), 0, st, p); break;
    case 128: hipLaunchKernelGGL(k_near<128>, grid, dim3(NEAR_THREADS), 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace swl
