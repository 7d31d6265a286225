/*
 * swl.h — sink + window + landmark ("sealed O(1)") attention on AMD MI355X
 * (gfx950).  C ABI of libswl.so.
 *
 * The layer: for every KV group g and query head h, a row attends under one
 * softmax to three sources — ns sink keys, a ring-buffer window of the last
 * w_g keys (self included), and a far field that summarises every key the
 * window has evicted.  The far field keeps, per query head and landmark b, a
 * running max M_b, a mass Z_b and a value accumulator Theta_b (an online
 * softmax of landmark query q~_b over the evicted keys), and is read through
 * the Nystrom estimate u_b = sum_a exp(f_a - f_max) mu[a][b] with
 * f_a = scale <q, k~_a>.  Source: cortiq-engine 0.8.51
 * src/gpu_wgpu/o1_batch.rs (module doc; kernels o1b_far_e, o1b_attend,
 * o1b_far_commit, o1b_ring_commit, o1b_meta) and cortiq-engine 0.8.82
 * src/gpu_metal/o1c.rs (encode, encode_tok, state_commit).
 *
 * Geometry (swl_geom): G KV groups, H query heads per group (nh = G*H,
 * query head gh = g*H + h), m landmarks, W ring stride (the widest group
 * window), ns sinks, d key width, dv value width, scale (usually 1/sqrt(d)),
 * rect (1: clamp u_b at 0).  Supported: d == dv in {8, 16, 32, 64, 128, 256},
 * 1 <= m <= 64, 1 <= H <= 16, 1 <= G <= 64, 0 <= ns <= 256, 1 <= W <= 65536;
 * anything else is SWL_EINVAL.  (The pages admit their batch kernels only
 * for w >= 64, ns <= 255, ns + w <= 2052 and m <= 32 -- o1_batch.rs
 * min_window, o1c.rs admits, dory.rs forward -- capacities of their
 * fixed-size workgroup arrays; these kernels stream keys through LDS tiles
 * and have no such arrays.)
 *
 * Input range.  The prefill path multiplies on fp16 matrix cores with
 * fp32-accurate hi/lo splits of its operands, so keys, landmark keys,
 * landmark queries and scale * log2(e) * q must have magnitudes of at most
 * 65504 (fp16's largest value); beyond that the split rounds to infinity
 * and the outputs are inf or NaN (inputs are not scanned for it).  Values
 * may have any finite magnitude: each pass scales them by a power of two
 * before their split.  The decode path computes in fp32 throughout.
 *
 * Device arrays (swl_state; all row-major, fp32 unless noted):
 *   meta    u32 [G][4]   len, head, nfar, window override (0 = W)
 *   ring_k  [G][W][d]    ring_v [G][W][dv]   logical key x of group g sits
 *                        in slot (head + x) mod w_g
 *   sink_k  [G][ns][d]   sink_v [G][ns][dv]
 *   k_tilde [G][m][d]    landmark keys
 *   q_tilde [nh][m][d]   landmark queries
 *   mu      [nh][m][m]   mu[gh][a][b]
 *   mz      [nh][2][m]   M (row 0) then Z (row 1); an empty far field is
 *                        M = -inf, Z = 0
 *   theta   [nh][m][dv]
 * Call arrays: q [rows][nh][d] (rotated), k [rows][G][d] (rotated),
 * v [rows][G][dv], out [rows][nh][dv].
 *
 * Ownership: the caller allocates every array, including the scratch
 * buffer, in device memory; the library allocates nothing, keeps no global
 * state and never frees.  Every call only enqueues kernels on `stream`
 * (a hipStream_t; NULL is the default stream) and returns; results are
 * ready when the stream is.  Calls on one state must be ordered on one
 * stream.
 *
 * Errors: every entry point validates its arguments on the host before it
 * enqueues anything; on SWL_EINVAL nothing was enqueued.  SWL_EHIP means a
 * launch failed (hipGetLastError); earlier launches of that call may have
 * run.
 */
#ifndef SWL_H
#define SWL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWL_OK 0
#define SWL_EINVAL 1
#define SWL_EHIP 2
#define SWL_ESIZE 3   /* swl_attend_token_noalloc: the geometry needs more scratch than it holds */

/* Bytes of the library's static scratch (swl_attend_token_noalloc). */
#define SWL_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)

/* Rows of one sub-chunk (the pages' OB_K): a chunk longer than this is
 * processed as consecutive sub-chunks of this many rows. */
#define SWL_SUB 64

typedef struct swl_geom {
    int32_t G, H, m, W, ns, d, dv;
    float scale;
    int32_t rect;
} swl_geom;

typedef struct swl_state {
    uint32_t* meta;
    float* ring_k;
    float* ring_v;
    const float* sink_k;
    const float* sink_v;
    const float* k_tilde;
    const float* q_tilde;
    const float* mu;
    float* mz;
    float* theta;
} swl_state;

/* Bytes of scratch a call over `rows` rows needs (attend_chunk + commit on
 * the same rows, prefill, or attend_token with rows = 1).  Prefill over
 * more rows than one pass holds reuses the scratch pass after pass, so the
 * size stops growing at 32768 rows.  Returns 0 for an invalid geometry. */
size_t swl_scratch_bytes(const swl_geom* geom, int64_t rows);

/* The empty state (o1b_meta's fields at zero pushes; o1b_far_e's empty far
 * field): meta[g] = {0, 0, 0, windows[g]}, M = -inf, Z = 0, Theta = 0.
 * `windows` is a host array of G window overrides (0 = W, else
 * 1 <= w_g <= W) or NULL for all W.  Sinks, landmarks and mu are the
 * caller's.  Ring contents are left as they are (len = 0). */
int swl_init_state(const swl_geom* geom, const swl_state* st,
                   const uint32_t* windows, void* stream);

/* Attention of one sub-chunk of 1 <= rows <= 64 rows from the state, into
 * out (o1b_far_e then o1b_attend): every evicted key is scored against
 * every landmark query, the far max jumps to its post-chunk value, and each
 * row reads the far field rescaled to it plus a causal in-chunk sum over the
 * rows evicted so far.  Does not change the state; leaves the far-field
 * quantities of the sub-chunk in `scratch` for swl_commit. */
int swl_attend_chunk(const swl_geom* geom, const swl_state* st,
                     const float* q, const float* k, const float* v, int32_t rows,
                     float* out, void* scratch, size_t scratch_bytes, void* stream);

/* The state after the rows of the preceding swl_attend_chunk (same k, v,
 * rows and scratch, nothing else on the state or the scratch in between;
 * the value the rows add to the far accumulator is already in the
 * scratch): far commit
 * (Theta <- R Theta + sum_j E_j v_evicted(j), M, Z; o1b_far_commit), ring
 * commit (row j to slot (head0 + len0 + j) mod w_g; o1b_ring_commit) and
 * meta (len, head, nfar after `rows` pushes; o1b_meta). */
int swl_commit(const swl_geom* geom, const swl_state* st,
               const float* k, const float* v, int32_t rows,
               void* scratch, size_t scratch_bytes, void* stream);

/* attend + commit over any number of rows (rows >= 0; 0 is a no-op), as
 * consecutive 64-row sub-chunks with each sub-chunk's semantics (its own
 * post-sub-chunk far max): the same result as looping swl_attend_chunk +
 * swl_commit, up to rounding (o1_batch.rs encode, whose loop runs the
 * chunk kernels over sub-chunks of OB_K rows).  Sub-chunks are batched
 * into few launches: passes of up to 32768 rows.  q, k, v and out hold the
 * rows in order; scratch: swl_scratch_bytes(geom, rows) bytes. */
int swl_prefill(const swl_geom* geom, const swl_state* st,
                const float* q, const float* k, const float* v, int64_t rows,
                float* out, void* scratch, size_t scratch_bytes, void* stream);

/* Stages of a call, as reported to a swl_stage_fn.  A prefill pass makes
 * five launches, reported in this order: far score (which also forms the
 * accumulator increments, dtheta), far scan (which also takes the values'
 * scale), theta scan (which also splits the key tiles), attend, ring
 * (which also updates meta).  A pass without attention (swl_commit_rows)
 * makes three: far score, far scan, and theta scan with the ring and meta.
 * SWL_STAGE_DTHETA, SWL_STAGE_META, SWL_STAGE_KV_SPLIT and
 * SWL_STAGE_VALUE_SCALE name parts of those launches and are not reported
 * on their own. */
enum swl_stage {
    SWL_STAGE_FAR_SCORE = 0,  /* evicted key x landmark scores */
    SWL_STAGE_FAR_SCAN = 1,   /* post-sub-chunk max, rescale and incoming mass */
    SWL_STAGE_DTHETA = 2,     /* exp mass, its prefix and the value added to the accumulator */
    SWL_STAGE_THETA_SCAN = 3, /* the accumulator before each sub-chunk; commit of M, Z, Theta */
    SWL_STAGE_ATTEND = 4,     /* sinks + window attention and the far readout */
    SWL_STAGE_RING = 5,       /* ring commit */
    SWL_STAGE_META = 6,       /* len, head, nfar */
    SWL_STAGE_KV_SPLIT = 7,   /* the pass's keys and values as fp16 hi/lo tiles */
    SWL_STAGE_VALUE_SCALE = 8, /* the largest |value| of the pass, per group */
    SWL_STAGE_COUNT = 9
};

/* Host callback invoked around each launch while the launches are being
 * enqueued: begin = 1 just before the launch of `stage`, begin = 0 just
 * after it.  Work the callback enqueues on the same stream (an event
 * record, for instance) is ordered between that launch and its
 * neighbours, which is how a caller times one stage on the GPU. */
typedef void (*swl_stage_fn)(int32_t stage, int32_t begin, void* user);

/* swl_prefill with a stage callback (fn may be NULL: then it is
 * swl_prefill). */
int swl_prefill_traced(const swl_geom* geom, const swl_state* st,
                       const float* q, const float* k, const float* v, int64_t rows,
                       float* out, void* scratch, size_t scratch_bytes, void* stream,
                       swl_stage_fn fn, void* user);

/* The state after `rows` rows (rows >= 0; 0 is a no-op) whose keys and
 * values are k [rows][G][d] and v [rows][G][dv], without their attention:
 * far_e and the commit of every consecutive 64-row sub-chunk (o1c.rs
 * spec_commit, which moves a layer over the accepted rows of a verify).
 * A verify is a swl_attend_chunk over up to 64 speculative rows, which
 * leaves the state as it was; committing the first r of them with this
 * call gives the state of r serial steps, the far max taken over the
 * accepted rows only.  The same state as swl_prefill over the rows, up to
 * rounding.  scratch: swl_scratch_bytes(geom, rows) bytes. */
int swl_commit_rows(const swl_geom* geom, const swl_state* st,
                    const float* k, const float* v, int64_t rows,
                    void* scratch, size_t scratch_bytes, void* stream);

/* A layer sealed from `rows` exact rows (dory.rs seal, with the landmarks,
 * mu and the sinks already in the state): the empty state (as
 * swl_init_state, with the same `windows`), then swl_commit_rows over the
 * rows, so the ring holds the last min(rows, w_g) of them and M, Z, Theta
 * summarise the rows before those.  scratch: swl_scratch_bytes(geom, rows)
 * bytes (none for rows == 0). */
int swl_seal(const swl_geom* geom, const swl_state* st, const uint32_t* windows,
             const float* k, const float* v, int64_t rows,
             void* scratch, size_t scratch_bytes, void* stream);

/* The bookkeeping of the last push undone in every group (dory.rs
 * dory_o1_back, for models that run a layer several times per row): a full
 * window moves its head back one slot and its far count down by one, a
 * partial one loses its newest row; an empty window is left alone.  The
 * ring's rows and M, Z, Theta are not restored. */
int swl_rewind(const swl_geom* geom, const swl_state* st, void* stream);

/* One row, attended and committed: a sub-chunk of one row (o1c.rs
 * encode_tok) in two launches.  The row's keys (sinks, then the window after
 * the push) are split over blocks of 64 keys per group, each writing a
 * partial (max, mass, value sum) for every head; alongside, each query
 * head's landmarks fold in the key the row evicts (when the ring is full)
 * and produce the far part.  A merge per group brings the partials to one
 * exponent, drops a far part whose mass is not >= 0, writes out, and pushes
 * the row into the ring.  Same result as attend_chunk + commit with
 * rows = 1, up to rounding. */
int swl_attend_token(const swl_geom* geom, const swl_state* st,
                     const float* q, const float* k, const float* v,
                     float* out, void* scratch, size_t scratch_bytes, void* stream);

/* Fused ingest and output steps (dory.rs page: the preparation kernel
 * dory_prep and the gate kernels dory_gate1 / dory_ogate), so that q and
 * the output make no pass of their own through memory:
 *   rope        [rows][d] floats, or NULL.  Row r holds cos of the d/2 pair
 *               angles of the call's row r, then their sin.  When set, q and
 *               k are the rows before RoPE: each kernel that reads a query
 *               or key head of row r turns its pair (j, j + d/2) into
 *               (x_j c_j - x_{j+d/2} s_j, x_{j+d/2} c_j + x_j s_j) in fp32,
 *               and the ring receives the turned keys.  Values are not
 *               turned.  (The page's kernel also normalises heads; that
 *               model-specific step is not part of this.)
 *   gate        [rows][G*H][dv] floats, or NULL: gate pre-activations z.
 *               When set, each output element is multiplied by
 *               1 / (1 + exp(-z s)) in fp32.
 *   gate_scale  [G*H][dv] floats: the scale s of each (head, column);
 *               required with gate (else SWL_EINVAL).
 * Device memory owned by the caller and only read.  Row 0 of rope and gate
 * is the call's first row (prefill advances them with its passes).  A NULL
 * swl_fuse pointer turns both steps off: each _fused call is then its
 * plain counterpart. */
typedef struct swl_fuse {
    const float* rope;
    const float* gate;
    const float* gate_scale;
} swl_fuse;

/* swl_prefill with the fused steps. */
int swl_prefill_fused(const swl_geom* geom, const swl_state* st,
                      const float* q, const float* k, const float* v, int64_t rows,
                      const swl_fuse* fuse, float* out, void* scratch,
                      size_t scratch_bytes, void* stream);

/* swl_attend_chunk with the fused steps (1 <= rows <= 64). */
int swl_attend_chunk_fused(const swl_geom* geom, const swl_state* st,
                           const float* q, const float* k, const float* v, int32_t rows,
                           const swl_fuse* fuse, float* out, void* scratch,
                           size_t scratch_bytes, void* stream);

/* swl_commit after swl_attend_chunk_fused: the same rope (the ring
 * receives the turned keys); the gate is not used. */
int swl_commit_fused(const swl_geom* geom, const swl_state* st,
                     const float* k, const float* v, int32_t rows, const swl_fuse* fuse,
                     void* scratch, size_t scratch_bytes, void* stream);

/* swl_commit_rows over keys before RoPE (the gate is not used). */
int swl_commit_rows_fused(const swl_geom* geom, const swl_state* st,
                          const float* k, const float* v, int64_t rows,
                          const swl_fuse* fuse, void* scratch, size_t scratch_bytes,
                          void* stream);

/* swl_attend_token with the fused steps (rope and gate of one row). */
int swl_attend_token_fused(const swl_geom* geom, const swl_state* st,
                           const float* q, const float* k, const float* v,
                           const swl_fuse* fuse, float* out, void* scratch,
                           size_t scratch_bytes, void* stream);

/* swl_attend_token_fused for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same kernels and results as swl_attend_token_fused (fuse
 * may be NULL: then swl_attend_token), but no scratch argument: the
 * decode partials go to a static device array of SWL_NOALLOC_SCRATCH_BYTES
 * bytes inside the library, one per GPU, which the first call on a GPU
 * looks up (hipGetSymbolAddress) and which stays allocated until the process
 * ends.  The call allocates nothing itself (no hipMalloc, no library routine
 * that allocates).  Geometries whose partials need more than that
 * (4 * ((G * ceil((ns + W) / 64) + 4 * G) * H * (dv + 4)) bytes) return
 * SWL_ESIZE before anything is enqueued.  Every call on one GPU shares that
 * GPU's array and each call overwrites what it reads, so calls that may
 * overlap on one GPU (other streams, other threads) race: order them on
 * one stream.  q, k, v, out and the state as in swl_attend_token. */
int swl_attend_token_noalloc(const swl_geom* geom, const swl_state* st,
                             const float* q, const float* k, const float* v,
                             const swl_fuse* fuse, float* out, void* stream);

/* A static description of a status code. */
const char* swl_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* SWL_H */
