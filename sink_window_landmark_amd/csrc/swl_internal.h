// Internal declarations of libswl: the parameter block every kernel takes,
// the closed-form ring bookkeeping, and the launchers the C entry points call.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/swl.h"

namespace swl {

constexpr int SUB = SWL_SUB;           // rows of a sub-chunk
constexpr int PASS_SUBS = 512;         // sub-chunks per prefill pass (32768 rows)
constexpr int VM_SLOTS = PASS_SUBS;     // value maxima per group (one per far_score block, <= 512)

// Everything a kernel of one call (or one prefill pass) needs, passed by value.
struct KParams {
    // geometry
    int G, H, m, W, ns, d, dv, nh, rect;
    float scale;
    // state (meta: the call-start bookkeeping; after a call's first launch it
    // points to the copy in scratch, meta_copy, so that the last launch can
    // write the new one to meta_out while others read the old)
    uint32_t* meta;
    uint32_t* meta_copy;      // [G][4] scratch copy of the call-start meta (written by far_score)
    uint32_t* meta_out;       // the state's meta (written by the meta update)
    float* ring_k;
    float* ring_v;
    const float* sink_k;
    const float* sink_v;
    const float* k_tilde;
    const float* q_tilde;
    const float* mu;
    float* mz;
    float* theta;
    // rows of this call / pass
    const float* q;
    const float* k;
    const float* v;
    float* out;
    int T;   // rows (<= PASS_SUBS * SUB)
    int S;   // sub-chunks, ceil(T / SUB)
    // scratch planes (see scratch_layout)
    float* E;    // [S][nh*m][SUB]  exp(l - mx_s) of the evicted keys' scores against the sub-chunk's own max (0: no eviction)
    float* FAC;  // [S][nh*m]       exp(mx_s - M'_s): E's factor to the post-sub-chunk max
    float* Ms;   // [S][nh*m]       local max of the scores, then the post-sub-chunk max
    float* Rs;   // [S][nh*m]       local mass of the scores, then the rescale of the old mass
    float* TZ;   // [S+1][nh*m]     mass before each sub-chunk, then after the last
    float* TH;   // [S][nh*m][dv]   Theta increments, then Theta before each sub-chunk
    const float* theta_prev;  // Theta before sub-chunk s at theta_prev + s*theta_prev_stride
    int64_t theta_prev_stride;
    float* apart;             // split-window attention partials (attend_part_floats())
    int nsp;                  // splits of the window per attention work item (set by launch_attend)
    int msplit;               // merge blocks split a head's query rows and landmarks (set by launch_attend)
    float* vmax;              // [G][VM_SLOTS] largest |value| seen by each far_score block of the group
    int vm_n;                 // value-maxima shares per group (slots of vmax in use)
    int vm_far;               // far_score takes the value maxima (no far scan launch follows)
    unsigned short* kvs;      // [G][kv_tiles] fp16 key tiles of the pass (k_kv_split)
    int kv_tiles;             // tiles per group: the sinks, then the aligned window tiles
    // fused ingest and output steps (null: off)
    const float* rope;        // [T][d] row r: cos of the d/2 pair angles, then their sin
    const float* gate;        // [T][nh][dv] gate pre-activations
    const float* gate_scale;  // [nh][dv]
};

// Elements c4 .. c4+3 of row x (a query or key head of D elements) after
// the rotate-half RoPE of table row tab (cos of the D/2 pair angles, then
// their sin): pair (j, j + D/2) becomes (x_j c - x_{j+D/2} s,
// x_{j+D/2} c + x_j s).  tab null: the elements as they are.  c4 a
// multiple of 4 and D of 8, so that a float4 never straddles the halves.
__device__ __forceinline__ float4 rope4(const float* x, const float* tab, int c4, int D)
{
    if (!tab) return *reinterpret_cast<const float4*>(x + c4);
    const int h = D >> 1;
    const bool first = c4 < h;
    const int j = first ? c4 : c4 - h;
    const float4 a = *reinterpret_cast<const float4*>(x + j);
    const float4 b = *reinterpret_cast<const float4*>(x + j + h);
    const float4 cs = *reinterpret_cast<const float4*>(tab + j);
    const float4 sn = *reinterpret_cast<const float4*>(tab + h + j);
    if (first)
        return make_float4(a.x * cs.x - b.x * sn.x, a.y * cs.y - b.y * sn.y, a.z * cs.z - b.z * sn.z,
                           a.w * cs.w - b.w * sn.w);
    return make_float4(b.x * cs.x + a.x * sn.x, b.y * cs.y + a.y * sn.y, b.z * cs.z + a.z * sn.z,
                       b.w * cs.w + a.w * sn.w);
}

// The output gate 1 / (1 + exp(-z s)), as 1 / (1 + 2^(-z s log2 e)) on the
// hardware exponential and reciprocal (a few ulp in all; 0 for very negative
// z s, 1 for very positive: the exponential overflows to inf or underflows
// to 0, no NaN).
__device__ __forceinline__ float gate_of(float z, float s)
{
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * s * 1.4426950408889634f));
}

// Ring bookkeeping of group g at the start of a call.
struct GMeta {
    int len0, head0, nfar0, wg;
};

__device__ __forceinline__ GMeta load_gmeta(const uint32_t* meta, int g, int W)
{
    GMeta c;
    c.len0 = (int)meta[4 * g + 0];
    c.head0 = (int)meta[4 * g + 1];
    c.nfar0 = (int)meta[4 * g + 2];
    uint32_t w = meta[4 * g + 3];
    c.wg = w ? (int)w : W;
    return c;
}

// Ring bookkeeping at the start of the sub-chunk that begins `r0` rows into
// the call: the closed form of r0 single pushes (o1b_meta applied r0 times).
struct SubMeta {
    int len0, head0, nfar0, j0;
};

__device__ __forceinline__ SubMeta sub_meta(const GMeta& c, int r0)
{
    SubMeta s;
    int tot = c.len0 + r0;
    int ev = tot > c.wg ? tot - c.wg : 0;
    s.len0 = tot < c.wg ? tot : c.wg;
    s.head0 = (c.head0 + ev) % c.wg;
    s.nfar0 = c.nfar0 + ev;
    s.j0 = c.wg - s.len0;
    return s;
}

// Key positions of a call count keys in push order: the call-start ring in
// logical order (positions 0 .. len0-1), then the call's rows.  Position p
// of group g lives in ring slot (head0 + p) mod w_g when p < len0, else in
// row p - len0 of the call's k/v.  Chunk row j of the sub-chunk at r0 is
// position len0 + r0 + j, and it evicts position len0 + r0 + j - w_g.
__device__ __forceinline__ const float* key_row(const KParams& p, const GMeta& c, int g, int pos)
{
    if (pos < c.len0) return p.ring_k + ((int64_t)g * p.W + (c.head0 + pos) % c.wg) * p.d;
    return p.k + ((int64_t)(pos - c.len0) * p.G + g) * p.d;
}

__device__ __forceinline__ const float* val_row(const KParams& p, const GMeta& c, int g, int pos)
{
    if (pos < c.len0) return p.ring_v + ((int64_t)g * p.W + (c.head0 + pos) % c.wg) * p.dv;
    return p.v + ((int64_t)(pos - c.len0) * p.G + g) * p.dv;
}

// Work item of linear workgroup b out of n when the hardware deals
// workgroups round-robin over the 8 XCDs (b goes to XCD b mod 8, each with
// its own L2): XCD x takes the contiguous run of work items
// [x*q + min(x, r), ...) with q = n / 8, r = n % 8, so neighbouring work
// items (which share keys) meet in the same L2.
__device__ __forceinline__ int xcd_work_item(int b, int n)
{
    const int x = b & 7, k = b >> 3;
    const int q = n >> 3, r = n & 7;
    return x * q + (x < r ? x : r) + k;
}

// The power-of-two scale of a group's values in a pass: with vmax the
// largest |value| among the pass's sinks, call-start window and rows, the
// values times 2^e have magnitudes below 2^14, so that both fp16 halves of
// their splits are normal numbers far inside fp16 range whatever the values'
// own scale (exact: a power of two; undone on the products' results).  0
// for no values, or when the largest is not finite (the results are then
// not finite either, as they would be without the scale).
__host__ __device__ inline int value_exp_of(float vmax)
{
    if (!(vmax > 0.f) || !(vmax <= 3.4028235e38f)) return 0;
    int ex;
    frexpf(vmax, &ex);   // vmax = f 2^ex, 0.5 <= f < 1
    return 14 - ex;
}

// Work item (s, gi, sp) at position pos of an order that splits the S
// sub-chunks into 8 contiguous ranges, one per XCD (xcd_work_item deals
// positions to XCDs in contiguous runs), then takes the NG groups (or
// (head group, group) pairs) of a range one after the other, then the
// sub-chunks of the range, then nsp splits of each.  Each XCD then runs an
// equal share of every group's sub-chunks, whatever the groups' windows,
// while the blocks it runs together still cover consecutive sub-chunks of
// one group (which share their key band in its L2).
__device__ __forceinline__ void range_item(int pos, int S, int NG, int nsp, int& s, int& gi, int& sp)
{
    const int per_s = NG * nsp, q = S >> 3, rem = S & 7;
    int lo = 0;
    s = gi = sp = 0;
    for (int r = 0; r < 8; ++r) {
        const int len = q + (r < rem ? 1 : 0);
        if (pos < (lo + len) * per_s) {
            const int local = pos - lo * per_s;
            sp = local % nsp;
            const int t = local / nsp;   // gi * len + (s - lo)
            s = lo + t % len;
            gi = t / len;
            return;
        }
        lo += len;
    }
}

// far_score: sub-chunks per block (FS_RUN while the launch keeps at least
// 256 blocks, fewer for short calls) and blocks per group
constexpr int FS_RUN = 4;
__host__ __device__ inline int fs_run(int S, int G)
{
    int rl = FS_RUN;
    while (rl > 1 && ((S + rl - 1) / rl) * G < 256) rl >>= 1;
    return rl;
}
// blocks per group of runs of sub-chunks
__host__ __device__ inline int fs_runs(int S, int G)
{
    const int rl = fs_run(S, G);
    return (S + rl - 1) / rl;
}
// blocks per run: while the launch would have fewer than 128 working
// blocks, the hm / 32 landmark-row tiles of a run are split over 2, 4, ...
// blocks (a power of two, at most the tile count).  Each such block loads
// the run's keys and values again, so launches that already fill half the
// machine keep one block per run.
__host__ __device__ inline int fs_tsplit(int S, int G, int hm)
{
    const int nht = (hm + 31) / 32;
    const int n = fs_runs(S, G) * G;
    int ts = 1;
    while (2 * ts <= nht && n * ts < 128) ts *= 2;
    return ts;
}
// value-maxima shares per group: one per far_score run and tile split, and
// at least 32 (the far scan launch's maxima blocks; a call without that
// launch gives far_score FS_MIN_BLOCKS maxima blocks per group of their own)
constexpr int FS_MIN_BLOCKS = 32;
__host__ __device__ inline int fs_blocks_per_group(int S, int G, int hm)
{
    const int n = fs_runs(S, G) * fs_tsplit(S, G, hm);
    return n > FS_MIN_BLOCKS ? n : FS_MIN_BLOCKS;
}

// Launchers (each returns the launch's hipGetLastError).
hipError_t launch_init(const KParams& p, const uint32_t* windows, hipStream_t st);
hipError_t launch_far_score(const KParams& p, hipStream_t st);
// the far scan and the accumulator increments in one launch
hipError_t launch_far_scan(const KParams& p, bool vm, hipStream_t st);   // vm: with the value maxima
// the accumulator scan (commit) and the key tiles in one launch (either may be off)
hipError_t launch_theta_kv(const KParams& p, bool mz, bool theta, bool kv, hipStream_t st);
hipError_t launch_attend(const KParams& p, hipStream_t st);
// tiles per group and bytes per tile of the fp16 key tiles
int kv_tiles(int ns, int W, int S);
size_t kv_tile_bytes(int d);
// floats of the split-window attention partials (a plane of fixed size: at
// most 256 (block, split) pairs of one launch)
size_t attend_part_floats(int d);
// the ring commit and the meta update, after the accumulator scan when `theta`
hipError_t launch_commit(const KParams& p, bool theta, hipStream_t st);
hipError_t launch_rewind(const KParams& p, hipStream_t st);
// one-row decode: partials, then merge + commit; `part` holds tok_part_floats()
hipError_t launch_token(const KParams& p, float* part, hipStream_t st);
size_t tok_part_floats(int G, int H, int dv, int ns, int W);

}  // namespace swl
