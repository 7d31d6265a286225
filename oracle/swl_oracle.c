/*
 * Serial CPU oracle of the sealed O(1) attention layer: sink keys, a ring
 * window of the last w_g keys, and a landmark far field.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library; the GPU library
 * never does, and this file shares no code, header or table with it.
 *
 * It steps one row at a time, in float64, in the order the pages state the
 * per-row spec (cortiq-engine o1_batch.rs module doc: the chunk kernels are
 * specified against the serial per-row step "step_group").  That serial step
 * is not printed on the pages; it is restated here from the chunk kernels of
 * o1_batch.rs (o1b_far_e, o1b_attend, o1b_far_commit, o1b_ring_commit,
 * o1b_meta) run with a chunk of one row:
 *
 *   push   (o1b_ring_commit, o1b_meta): the row's key and value enter the
 *          ring.  While len < w_g the slot is (head + len) mod w_g and len
 *          grows; once the ring is full the slot is head, the key there is
 *          evicted first, head advances and nfar grows.
 *   evict  (o1b_far_e, o1b_far_commit): for every query head h and landmark
 *          b, l = scale * <q~_hb, k_e>; M' = max(M, l); R = 1 when M' == M
 *          (so an empty field at -inf never forms -inf - -inf), otherwise
 *          exp(M - M'); Z <- R Z + exp(l - M'); Theta <- R Theta +
 *          exp(l - M') v_e; M <- M'.
 *   attend (o1b_attend): scores over the sinks and the window (self
 *          included); if nfar > 0 the Nystrom far estimate joins under one
 *          exponent: f_a = scale <q, k~_a>, u_b = sum_a exp(f_a - fmax)
 *          mu[a][b] (clamped at 0 when rect), c = max(c_near, max_b fmax +
 *          M_b), gain_b = u_b exp(fmax + M_b - c), D_far = sum_b gain_b Z_b,
 *          N_far = sum_b gain_b Theta_b; a D_far that is not >= 0 (negative
 *          or NaN) drops both.  out = (N_far + sum p v) /
 *          max(D_far + sum p, 1e-30) with p = exp(s - c).
 *
 * Build: gcc -O2 -shared -fPIC swl_oracle.c -o libswl_oracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t H, m, W, wg, ns, d, dv, rect;
    double scale;
    int32_t h_lo, h_hi; /* query heads this call attends and whose far state it updates */
} swlo_geom;

typedef struct {
    int64_t* meta;        /* len, head, nfar */
    double* ring_k;       /* [W][d]   (slots >= wg unused) */
    double* ring_v;       /* [W][dv] */
    const double* sink_k; /* [ns][d] */
    const double* sink_v; /* [ns][dv] */
    const double* k_tilde;/* [m][d] */
    const double* q_tilde;/* [H][m][d] */
    const double* mu;     /* [H][m][m], mu[h][a][b] */
    double* M;            /* [H][m] */
    double* Z;            /* [H][m] */
    double* theta;        /* [H][m][dv] */
} swlo_state;

static double dot_dd(const double* a, const double* b, int n)
{
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += a[i] * b[i];
    return s;
}

static double dot_fd(const float* a, const double* b, int n)
{
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += (double)a[i] * b[i];
    return s;
}

/* Fold the evicted key/value into every landmark summary of heads [h_lo, h_hi). */
static void evict(const swlo_geom* g, swlo_state* st, const double* ke, const double* ve)
{
    for (int h = g->h_lo; h < g->h_hi; ++h) {
        for (int b = 0; b < g->m; ++b) {
            const double* qt = st->q_tilde + ((int64_t)h * g->m + b) * g->d;
            double l = g->scale * dot_dd(qt, ke, g->d);
            double* Mp = st->M + (int64_t)h * g->m + b;
            double* Zp = st->Z + (int64_t)h * g->m + b;
            double* th = st->theta + ((int64_t)h * g->m + b) * g->dv;
            double m_old = *Mp;
            double m_new = l > m_old ? l : m_old;
            double R = (m_new == m_old) ? 1.0 : exp(m_old - m_new);
            double e = exp(l - m_new);
            *Zp = *Zp * R + e;
            for (int t = 0; t < g->dv; ++t) th[t] = th[t] * R + e * ve[t];
            *Mp = m_new;
        }
    }
}

/* Attention output of one query head for the current window and far field. */
static void attend(const swlo_geom* g, const swlo_state* st, int h, const float* q,
                   double* out, double* sc, double* fa, double* ub, double* nfar_v)
{
    const int64_t len = st->meta[0], head = st->meta[1], nfar = st->meta[2];
    const int ns = g->ns, d = g->d, dv = g->dv, m = g->m;
    const int64_t n = ns + len;
    double c = -INFINITY;
    for (int64_t x = 0; x < n; ++x) {
        const double* key;
        if (x < ns) key = st->sink_k + x * d;
        else key = st->ring_k + ((head + (x - ns)) % g->wg) * d;
        sc[x] = g->scale * dot_fd(q, key, d);
        if (sc[x] > c) c = sc[x];
    }
    double d_far = 0.0;
    for (int t = 0; t < dv; ++t) nfar_v[t] = 0.0;
    if (nfar > 0) {
        double fmax = -INFINITY;
        for (int a = 0; a < m; ++a) {
            fa[a] = g->scale * dot_fd(q, st->k_tilde + (int64_t)a * d, d);
            if (fa[a] > fmax) fmax = fa[a];
        }
        const double* mu = st->mu + (int64_t)h * m * m;
        for (int b = 0; b < m; ++b) {
            double u = 0.0;
            for (int a = 0; a < m; ++a) u += exp(fa[a] - fmax) * mu[(int64_t)a * m + b];
            if (g->rect && u < 0.0) u = 0.0;
            ub[b] = u;
        }
        const double* Mh = st->M + (int64_t)h * m;
        const double* Zh = st->Z + (int64_t)h * m;
        for (int b = 0; b < m; ++b)
            if (fmax + Mh[b] > c) c = fmax + Mh[b];
        for (int b = 0; b < m; ++b) {
            double gain = ub[b] * exp(fmax + Mh[b] - c);
            d_far += gain * Zh[b];
            const double* th = st->theta + ((int64_t)h * m + b) * dv;
            for (int t = 0; t < dv; ++t) nfar_v[t] += gain * th[t];
        }
        if (!(d_far >= 0.0)) {
            d_far = 0.0;
            for (int t = 0; t < dv; ++t) nfar_v[t] = 0.0;
        }
    }
    double den = d_far;
    for (int t = 0; t < dv; ++t) out[t] = nfar_v[t];
    for (int64_t x = 0; x < n; ++x) {
        double p = exp(sc[x] - c);
        den += p;
        const double* val;
        if (x < ns) val = st->sink_v + x * dv;
        else val = st->ring_v + ((head + (x - ns)) % g->wg) * dv;
        for (int t = 0; t < dv; ++t) out[t] += p * val[t];
    }
    if (den < 1e-30) den = 1e-30;
    for (int t = 0; t < dv; ++t) out[t] /= den;
}

/*
 * Step `rows` rows of one KV group.
 *   q   row r, head h at q + r*q_stride + h*d   (h is the group-local head)
 *   k   row r at k + r*k_stride;  v likewise
 *   out row r, head h at out + slot*out_stride + h*dv where slot =
 *       out_slot[r] (NULL: slot = r); a negative slot skips the attention
 *       of that row (the state still advances).
 * Returns 0, or -1 on a bad argument.
 */
int swlo_step_rows(const swlo_geom* g, swlo_state* st, int64_t rows,
                   const float* q, int64_t q_stride,
                   const float* k, int64_t k_stride,
                   const float* v, int64_t v_stride,
                   double* out, int64_t out_stride, const int64_t* out_slot)
{
    if (!g || !st || g->wg < 1 || g->wg > g->W || g->h_lo < 0 || g->h_hi > g->H ||
        g->h_lo > g->h_hi || g->m < 1 || g->d < 1 || g->dv < 1 || g->ns < 0)
        return -1;
    const int d = g->d, dv = g->dv;
    double* sc = malloc(sizeof(double) * (size_t)(g->ns + g->wg));
    double* fa = malloc(sizeof(double) * (size_t)g->m);
    double* ub = malloc(sizeof(double) * (size_t)g->m);
    double* nv = malloc(sizeof(double) * (size_t)dv);
    double* ke = malloc(sizeof(double) * (size_t)d);
    double* ve = malloc(sizeof(double) * (size_t)dv);
    if (!sc || !fa || !ub || !nv || !ke || !ve) {
        free(sc); free(fa); free(ub); free(nv); free(ke); free(ve);
        return -1;
    }
    for (int64_t r = 0; r < rows; ++r) {
        const float* kr = k + r * k_stride;
        const float* vr = v + r * v_stride;
        int64_t len = st->meta[0], head = st->meta[1];
        int64_t slot;
        if (len < g->wg) {
            slot = (head + len) % g->wg;
            st->meta[0] = len + 1;
        } else {
            slot = head;
            memcpy(ke, st->ring_k + slot * d, sizeof(double) * (size_t)d);
            memcpy(ve, st->ring_v + slot * dv, sizeof(double) * (size_t)dv);
            evict(g, st, ke, ve);
            st->meta[1] = (head + 1) % g->wg;
            st->meta[2] += 1;
        }
        for (int t = 0; t < d; ++t) st->ring_k[slot * d + t] = (double)kr[t];
        for (int t = 0; t < dv; ++t) st->ring_v[slot * dv + t] = (double)vr[t];

        int64_t os = out_slot ? out_slot[r] : r;
        if (out && os >= 0) {
            for (int h = g->h_lo; h < g->h_hi; ++h)
                attend(g, st, h, q + r * q_stride + (int64_t)h * d,
                       out + os * out_stride + (int64_t)h * dv, sc, fa, ub, nv);
        }
    }
    free(sc); free(fa); free(ub); free(nv); free(ke); free(ve);
    return 0;
}
