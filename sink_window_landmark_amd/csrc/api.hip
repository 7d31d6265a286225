// C entry points of libswl: host-side validation, scratch carving and the
// launch sequence of each call.  Launch order per sub-chunk follows the
// pages' encoder (cortiq-engine 0.8.51 src/gpu_wgpu/o1_batch.rs, encode:
// far_e, attend, far_commit, ring_commit, meta): the far commit must follow
// every read of the old accumulator, and the ring commit every read of the
// evicted rows.  A prefill pass runs the same steps over up to 512
// sub-chunks per launch.
#include <math.h>
#include <string.h>

#include <mutex>

#include "swl_internal.h"

namespace swl {

// Scratch of swl_attend_token_noalloc: file-scope device memory of a fixed
// size.  Every GPU the library runs on holds its own copy, at its own
// address, until the process ends.  In host code the array's name is only a
// stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, once per device (noalloc_scratch below), and only
// that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[SWL_NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEV = 64;
static std::mutex noalloc_mu;
static void* noalloc_addr[NOALLOC_MAX_DEV];

// This stream's GPU's copy of `scratch` (NULL stream: the current GPU), its
// address taken with that GPU current on the first call there; null on a
// HIP error.
static void* noalloc_scratch(hipStream_t stream)
{
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    int dev = cur;
    if (stream) {
        hipDevice_t d;
        if (hipStreamGetDevice(stream, &d) != hipSuccess) return nullptr;
        dev = (int)d;
    }
    if (dev < 0 || dev >= NOALLOC_MAX_DEV) return nullptr;
    std::lock_guard<std::mutex> lock(noalloc_mu);
    if (!noalloc_addr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return nullptr;
        void* addr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return nullptr;
        if (e != hipSuccess || !addr) return nullptr;
        noalloc_addr[dev] = addr;
    }
    return noalloc_addr[dev];
}

static bool geom_ok(const swl_geom* g)
{
    if (!g) return false;
    if (g->G < 1 || g->G > 64) return false;
    if (g->H < 1 || g->H > 16) return false;
    if (g->m < 1 || g->m > 64) return false;
    if (g->W < 1 || g->W > 65536) return false;
    if (g->ns < 0 || g->ns > 256) return false;
    if (g->d != g->dv) return false;
    if (!(g->d == 8 || g->d == 16 || g->d == 32 || g->d == 64 || g->d == 128 || g->d == 256)) return false;
    if (!isfinite(g->scale)) return false;
    if (g->rect != 0 && g->rect != 1) return false;
    return true;
}

static bool state_ok(const swl_geom* g, const swl_state* st)
{
    if (!st) return false;
    if (!st->meta || !st->ring_k || !st->ring_v || !st->k_tilde || !st->q_tilde || !st->mu ||
        !st->mz || !st->theta)
        return false;
    if (g->ns > 0 && (!st->sink_k || !st->sink_v)) return false;
    return true;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Carve {
    size_t tok, apart, mc, vm, e, fac, ms, rs, tz, th, kv, total;
};

static Carve carve(const swl_geom* g, int S)
{
    const size_t nhm = (size_t)g->G * g->H * g->m;
    Carve c;
    size_t off = 0;
    // the decode plane comes first, at an offset that does not depend on S
    c.tok = off; off += align256(sizeof(float) * tok_part_floats(g->G, g->H, g->dv, g->ns, g->W));
    c.apart = off; off += align256(sizeof(float) * attend_part_floats(g->d));
    c.mc = off; off += align256(sizeof(uint32_t) * 4 * (size_t)g->G);
    c.vm = off; off += align256(sizeof(float) * (size_t)g->G * VM_SLOTS);
    c.e = off;  off += align256(sizeof(float) * (size_t)S * nhm * SUB);
    c.fac = off; off += align256(sizeof(float) * (size_t)S * nhm);
    c.ms = off; off += align256(sizeof(float) * (size_t)S * nhm);
    c.rs = off; off += align256(sizeof(float) * (size_t)S * nhm);
    c.tz = off; off += align256(sizeof(float) * (size_t)(S + 1) * nhm);
    c.th = off; off += align256(sizeof(float) * (size_t)S * nhm * g->dv);
    c.kv = off; off += align256((size_t)g->G * kv_tiles(g->ns, g->W, S) * kv_tile_bytes(g->d));
    c.total = off;
    return c;
}

static int subs_for_rows(int64_t rows)
{
    int64_t r = rows < 1 ? 1 : rows;
    int64_t cap = (int64_t)PASS_SUBS * SUB;
    if (r > cap) r = cap;
    return (int)((r + SUB - 1) / SUB);
}

static KParams make_params(const swl_geom* g, const swl_state* st)
{
    KParams p;
    memset(&p, 0, sizeof(p));
    p.G = g->G; p.H = g->H; p.m = g->m; p.W = g->W; p.ns = g->ns;
    p.d = g->d; p.dv = g->dv; p.nh = g->G * g->H; p.rect = g->rect;
    p.scale = g->scale;
    p.meta = st->meta; p.meta_out = st->meta; p.ring_k = st->ring_k; p.ring_v = st->ring_v;
    p.sink_k = st->sink_k; p.sink_v = st->sink_v; p.k_tilde = st->k_tilde;
    p.q_tilde = st->q_tilde; p.mu = st->mu; p.mz = st->mz; p.theta = st->theta;
    return p;
}

static void set_scratch(KParams& p, const swl_geom* g, void* scratch, int S)
{
    Carve c = carve(g, S);
    char* b = static_cast<char*>(scratch);
    p.E = reinterpret_cast<float*>(b + c.e);
    p.FAC = reinterpret_cast<float*>(b + c.fac);
    p.Ms = reinterpret_cast<float*>(b + c.ms);
    p.Rs = reinterpret_cast<float*>(b + c.rs);
    p.TZ = reinterpret_cast<float*>(b + c.tz);
    p.TH = reinterpret_cast<float*>(b + c.th);
    p.apart = reinterpret_cast<float*>(b + c.apart);
    p.vmax = reinterpret_cast<float*>(b + c.vm);
    p.vm_n = fs_blocks_per_group(S, g->G, g->H * g->m);
    p.meta_copy = reinterpret_cast<uint32_t*>(b + c.mc);
    p.kvs = reinterpret_cast<unsigned short*>(b + c.kv);
    p.kv_tiles = kv_tiles(g->ns, g->W, S);
}

// The fused ingest/output pointers of a call whose rows start `row0` rows
// into the caller's arrays (null fuse: both steps off).
static bool fuse_ok(const swl_fuse* f) { return !f || !f->gate || f->gate_scale; }
static void set_fuse(KParams& p, const swl_fuse* f, int64_t row0)
{
    if (!f) return;
    if (f->rope) p.rope = f->rope + row0 * p.d;
    if (f->gate) p.gate = f->gate + row0 * p.nh * p.dv;
    p.gate_scale = f->gate_scale;
}

#define SWL_TRY(x)                          \
    do {                                    \
        if ((x) != hipSuccess) return SWL_EHIP; \
    } while (0)

// The launches after a call's first one read the call-start meta from its
// copy in scratch (far_score wrote it), so that the last one can update the
// state's meta while others read the old.
static KParams after_first(const KParams& p)
{
    KParams q = p;
    q.meta = p.meta_copy;
    return q;
}

// far_e (the values' scale, scores, E and the accumulator increment; then
// the far scan, beside the key tiles) + attention (near part and far
// readout) of one call; the state is unchanged.
static int run_attend(const KParams& p0, hipStream_t st)
{
    KParams p = p0;
    p.vm_far = 1;
    p.vm_n = FS_MIN_BLOCKS;   // far_score's value-maxima blocks per group
    SWL_TRY(launch_far_score(p, st));
    const KParams q = after_first(p);
    SWL_TRY(launch_theta_kv(q, true, false, true, st));
    SWL_TRY(launch_attend(q, st));
    return SWL_OK;
}

// far commit + ring commit + meta of one call (after run_attend on its rows,
// whose scratch holds the call-start meta), in one launch.
static int run_commit(const KParams& p, hipStream_t st)
{
    SWL_TRY(launch_commit(after_first(p), true, st));
    return SWL_OK;
}

}  // namespace swl

using namespace swl;

extern "C" {

size_t swl_scratch_bytes(const swl_geom* geom, int64_t rows)
{
    if (!geom_ok(geom) || rows < 0) return 0;
    return carve(geom, subs_for_rows(rows)).total;
}

int swl_init_state(const swl_geom* geom, const swl_state* st, const uint32_t* windows,
                   void* stream)
{
    if (!geom_ok(geom) || !state_ok(geom, st)) return SWL_EINVAL;
    if (windows) {
        for (int g = 0; g < geom->G; ++g)
            if (windows[g] > (uint32_t)geom->W) return SWL_EINVAL;
    }
    KParams p = make_params(geom, st);
    SWL_TRY(launch_init(p, windows, static_cast<hipStream_t>(stream)));
    return SWL_OK;
}

int swl_attend_chunk_fused(const swl_geom* geom, const swl_state* st, const float* q,
                           const float* k, const float* v, int32_t rows, const swl_fuse* fuse,
                           float* out, void* scratch, size_t scratch_bytes, void* stream)
{
    if (!geom_ok(geom) || !state_ok(geom, st) || !fuse_ok(fuse)) return SWL_EINVAL;
    if (rows < 1 || rows > SUB || !q || !k || !v || !out || !scratch) return SWL_EINVAL;
    if (scratch_bytes < carve(geom, 1).total) return SWL_EINVAL;
    KParams p = make_params(geom, st);
    p.q = q; p.k = k; p.v = v; p.out = out;
    set_fuse(p, fuse, 0);
    p.T = rows; p.S = 1;
    set_scratch(p, geom, scratch, 1);
    p.theta_prev = st->theta;
    p.theta_prev_stride = 0;
    return run_attend(p, static_cast<hipStream_t>(stream));
}

int swl_attend_chunk(const swl_geom* geom, const swl_state* st, const float* q, const float* k,
                     const float* v, int32_t rows, float* out, void* scratch,
                     size_t scratch_bytes, void* stream)
{
    return swl_attend_chunk_fused(geom, st, q, k, v, rows, nullptr, out, scratch, scratch_bytes,
                                  stream);
}

int swl_commit_fused(const swl_geom* geom, const swl_state* st, const float* k, const float* v,
                     int32_t rows, const swl_fuse* fuse, void* scratch, size_t scratch_bytes,
                     void* stream)
{
    if (!geom_ok(geom) || !state_ok(geom, st) || !fuse_ok(fuse)) return SWL_EINVAL;
    if (rows < 1 || rows > SUB || !k || !v || !scratch) return SWL_EINVAL;
    if (scratch_bytes < carve(geom, 1).total) return SWL_EINVAL;
    KParams p = make_params(geom, st);
    p.k = k; p.v = v;
    p.T = rows; p.S = 1;
    set_fuse(p, fuse, 0);
    set_scratch(p, geom, scratch, 1);
    return run_commit(p, static_cast<hipStream_t>(stream));
}

int swl_commit(const swl_geom* geom, const swl_state* st, const float* k, const float* v,
               int32_t rows, void* scratch, size_t scratch_bytes, void* stream)
{
    return swl_commit_fused(geom, st, k, v, rows, nullptr, scratch, scratch_bytes, stream);
}

}  // extern "C"

// Consecutive 64-row sub-chunks of `rows` rows, batched into passes of up
// to PASS_SUBS sub-chunks: far_e, far commit, (attention,) ring commit and
// meta of each pass, in five launches (three without `attend`, where q and
// out are not used).
static int run_rows(const swl_geom* geom, const swl_state* st, const float* q, const float* k,
                    const float* v, int64_t rows, const swl_fuse* fuse, float* out, void* scratch,
                    size_t scratch_bytes, void* stream, swl_stage_fn fn, void* user, bool attend)
{
    if (!geom_ok(geom) || !state_ok(geom, st) || !fuse_ok(fuse)) return SWL_EINVAL;
    if (rows < 0) return SWL_EINVAL;
    if (rows == 0) return SWL_OK;
    if (!k || !v || !scratch || (attend && (!q || !out))) return SWL_EINVAL;
    const int S_max = subs_for_rows(rows);
    if (scratch_bytes < carve(geom, S_max).total) return SWL_EINVAL;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const int64_t cap = (int64_t)PASS_SUBS * SUB;
    const int nh = geom->G * geom->H;
#define SWL_STAGE(id, launch)                   \
    do {                                        \
        if (fn) fn(id, 1, user);                \
        hipError_t e_ = (launch);               \
        if (fn) fn(id, 0, user);                \
        if (e_ != hipSuccess) return SWL_EHIP;  \
    } while (0)
    for (int64_t done = 0; done < rows;) {
        const int64_t T = rows - done < cap ? rows - done : cap;
        KParams p = make_params(geom, st);
        if (attend) {
            p.q = q + done * nh * geom->d;
            p.out = out + done * nh * geom->dv;
        }
        p.k = k + done * geom->G * geom->d;
        p.v = v + done * geom->G * geom->dv;
        set_fuse(p, fuse, done);
        p.T = (int)T;
        p.S = (int)((T + SUB - 1) / SUB);
        set_scratch(p, geom, scratch, S_max);
        p.theta_prev = p.TH;
        p.theta_prev_stride = (int64_t)nh * geom->m * geom->dv;
        SWL_STAGE(SWL_STAGE_FAR_SCORE, launch_far_score(p, hs));   // with the increments
        const KParams q = after_first(p);
        SWL_STAGE(SWL_STAGE_FAR_SCAN, launch_far_scan(q, attend, hs));   // with the values' scale
        if (attend) {
            SWL_STAGE(SWL_STAGE_THETA_SCAN, launch_theta_kv(q, false, true, true, hs));   // with the key tiles
            SWL_STAGE(SWL_STAGE_ATTEND, launch_attend(q, hs));
            SWL_STAGE(SWL_STAGE_RING, launch_commit(q, false, hs));   // with the meta
        } else {
            SWL_STAGE(SWL_STAGE_THETA_SCAN, launch_commit(q, true, hs));   // with ring and meta
        }
        done += T;
    }
#undef SWL_STAGE
    return SWL_OK;
}

extern "C" {

int swl_prefill_traced(const swl_geom* geom, const swl_state* st, const float* q,
                       const float* k, const float* v, int64_t rows, float* out, void* scratch,
                       size_t scratch_bytes, void* stream, swl_stage_fn fn, void* user)
{
    return run_rows(geom, st, q, k, v, rows, nullptr, out, scratch, scratch_bytes, stream, fn,
                    user, true);
}

int swl_prefill(const swl_geom* geom, const swl_state* st, const float* q, const float* k,
                const float* v, int64_t rows, float* out, void* scratch, size_t scratch_bytes,
                void* stream)
{
    return run_rows(geom, st, q, k, v, rows, nullptr, out, scratch, scratch_bytes, stream,
                    nullptr, nullptr, true);
}

int swl_prefill_fused(const swl_geom* geom, const swl_state* st, const float* q, const float* k,
                      const float* v, int64_t rows, const swl_fuse* fuse, float* out,
                      void* scratch, size_t scratch_bytes, void* stream)
{
    return run_rows(geom, st, q, k, v, rows, fuse, out, scratch, scratch_bytes, stream, nullptr,
                    nullptr, true);
}

int swl_commit_rows(const swl_geom* geom, const swl_state* st, const float* k, const float* v,
                    int64_t rows, void* scratch, size_t scratch_bytes, void* stream)
{
    return run_rows(geom, st, nullptr, k, v, rows, nullptr, nullptr, scratch, scratch_bytes,
                    stream, nullptr, nullptr, false);
}

int swl_commit_rows_fused(const swl_geom* geom, const swl_state* st, const float* k,
                          const float* v, int64_t rows, const swl_fuse* fuse, void* scratch,
                          size_t scratch_bytes, void* stream)
{
    return run_rows(geom, st, nullptr, k, v, rows, fuse, nullptr, scratch, scratch_bytes, stream,
                    nullptr, nullptr, false);
}

int swl_seal(const swl_geom* geom, const swl_state* st, const uint32_t* windows, const float* k,
             const float* v, int64_t rows, void* scratch, size_t scratch_bytes, void* stream)
{
    if (!geom_ok(geom) || !state_ok(geom, st)) return SWL_EINVAL;
    if (rows < 0) return SWL_EINVAL;
    if (rows > 0 && (!k || !v || !scratch || scratch_bytes < carve(geom, subs_for_rows(rows)).total))
        return SWL_EINVAL;
    const int rc = swl_init_state(geom, st, windows, stream);
    if (rc != SWL_OK) return rc;
    return swl_commit_rows(geom, st, k, v, rows, scratch, scratch_bytes, stream);
}

int swl_rewind(const swl_geom* geom, const swl_state* st, void* stream)
{
    if (!geom_ok(geom) || !state_ok(geom, st)) return SWL_EINVAL;
    KParams p = make_params(geom, st);
    SWL_TRY(launch_rewind(p, static_cast<hipStream_t>(stream)));
    return SWL_OK;
}

int swl_attend_token_fused(const swl_geom* geom, const swl_state* st, const float* q,
                           const float* k, const float* v, const swl_fuse* fuse, float* out,
                           void* scratch, size_t scratch_bytes, void* stream)
{
    if (!geom_ok(geom) || !state_ok(geom, st) || !fuse_ok(fuse)) return SWL_EINVAL;
    if (!q || !k || !v || !out || !scratch) return SWL_EINVAL;
    const Carve cv = carve(geom, 1);
    if (scratch_bytes < cv.total) return SWL_EINVAL;
    KParams p = make_params(geom, st);
    p.q = q; p.k = k; p.v = v; p.out = out;
    p.T = 1; p.S = 1;
    set_fuse(p, fuse, 0);
    float* part = reinterpret_cast<float*>(static_cast<char*>(scratch) + cv.tok);
    SWL_TRY(launch_token(p, part, static_cast<hipStream_t>(stream)));
    return SWL_OK;
}

int swl_attend_token(const swl_geom* geom, const swl_state* st, const float* q, const float* k,
                     const float* v, float* out, void* scratch, size_t scratch_bytes,
                     void* stream)
{
    return swl_attend_token_fused(geom, st, q, k, v, nullptr, out, scratch, scratch_bytes, stream);
}

int swl_attend_token_noalloc(const swl_geom* geom, const swl_state* st, const float* q,
                             const float* k, const float* v, const swl_fuse* fuse, float* out,
                             void* stream)
{
    if (!geom_ok(geom) || !state_ok(geom, st) || !fuse_ok(fuse)) return SWL_EINVAL;
    if (!q || !k || !v || !out) return SWL_EINVAL;
    const size_t need = sizeof(float) * tok_part_floats(geom->G, geom->H, geom->dv, geom->ns, geom->W);
    if (need > SWL_NOALLOC_SCRATCH_BYTES) return SWL_ESIZE;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    void* part = noalloc_scratch(hs);
    if (!part) return SWL_EHIP;
    KParams p = make_params(geom, st);
    p.q = q; p.k = k; p.v = v; p.out = out;
    p.T = 1; p.S = 1;
    set_fuse(p, fuse, 0);
    SWL_TRY(launch_token(p, static_cast<float*>(part), hs));
    return SWL_OK;
}

const char* swl_status_str(int status)
{
    switch (status) {
    case SWL_OK: return "ok";
    case SWL_EINVAL: return "invalid argument";
    case SWL_EHIP: return "HIP launch failed";
    case SWL_ESIZE: return "the geometry needs more than the static scratch (SWL_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

}  // extern "C"
