/*
 * oracle.c -- plain fp64 CPU reference of the MoE-layer hot path.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library. The HIP library never
 * links it, and it shares no code, header or table with the HIP kernels.
 *
 * Every function is the plain definition of one step, written as simple
 * loops. Integers are exact; floating point is evaluated in double precision
 * from the exact input values (fp32, or bf16 widened exactly), with no
 * intermediate rounding to a narrower type. OpenMP only splits independent
 * output rows across threads; the arithmetic of each output is a fixed
 * sequential loop.
 *
 * Sources (the pages this build follows):
 *  - Zyphra correlated expert placement / token shuffling page, English
 *    abstract: an MoE layer replaces the Transformer FFN with E expert
 *    networks and sends each token to k of them; expert parallelism spreads
 *    experts over GPUs; an all-to-all dispatches tokens to their experts and
 *    a second one combines the results; correlated placement puts experts
 *    that are often chosen together on one GPU; the dispatcher sends each
 *    token to each GPU once; neither method alters routing or parameters.
 *  - Cobalt page, English abstract: experts are co-activated when a single
 *    token selects both of them.
 * Readings where the pages are silent (softmax over the k selected logits,
 * tie order, group score, slot order, SwiGLU expert form, gate applied in
 * the combine) are listed with each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1

int orc_version(void) { return 1; }

/* Threads the parallel loops use. */
int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Exact widening of one stored element to double. */
static double orc_elem(const void* base, size_t i, int dt)
{
    if (dt == ORC_F32) return (double)((const float*)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* a precedes b in the routing order: larger logit first, lower index on a
 * tie. IEEE comparison, so -0 and +0 tie. */
static int orc_precedes(double la, int ia, double lb, int ib)
{
    return la > lb || (la == lb && ia < ib);
}

/*
 * Route one batch of tokens.
 * Each token is sent to k of the E experts (Zyphra page, English abstract).
 * Readings: the k experts with the largest logits are chosen, ties going to
 * the lower expert index, listed in that order; the gate weights are the
 * softmax of the k chosen logits, so they sum to one.
 * Group-limited variant (n_groups > 1): experts form n_groups contiguous
 * groups of E/n_groups; a group's score is its largest logit; only the
 * topk_groups best groups (ties to the lower group index) stay eligible.
 * Returns 0, or -1 on bad arguments / fewer than k eligible experts.
 */
int orc_route(const float* logits, int T, int E, int k, int n_groups, int topk_groups,
              int32_t* topk_idx, double* gates)
{
    if (T < 0 || E < 1 || k < 1 || k > E || n_groups < 1 || E % n_groups ||
        topk_groups < 1 || topk_groups > n_groups || topk_groups * (E / n_groups) < k)
        return -1;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int t = 0; t < T; ++t) {
        const float* l = logits + (size_t)t * E;
        char* eligible = (char*)malloc((size_t)E);
        char* taken = (char*)malloc((size_t)E);
        int gsz = E / n_groups;
        for (int e = 0; e < E; ++e) { eligible[e] = 1; taken[e] = 0; }
        if (n_groups > 1) {
            double* score = (double*)malloc(sizeof(double) * (size_t)n_groups);
            char* keep = (char*)calloc((size_t)n_groups, 1);
            for (int m = 0; m < n_groups; ++m) {
                double s = (double)l[m * gsz];
                for (int e = m * gsz + 1; e < (m + 1) * gsz; ++e)
                    if ((double)l[e] > s) s = (double)l[e];
                score[m] = s;
            }
            /* take the best remaining group topk_groups times */
            for (int r = 0; r < topk_groups; ++r) {
                int best = -1;
                for (int m = 0; m < n_groups; ++m)
                    if (!keep[m] && (best < 0 || orc_precedes(score[m], m, score[best], best)))
                        best = m;
                keep[best] = 1;
            }
            for (int e = 0; e < E; ++e) eligible[e] = keep[e / gsz];
            free(score);
            free(keep);
        }
        /* take the best remaining eligible expert k times */
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (eligible[e] && !taken[e] &&
                    (best < 0 || orc_precedes((double)l[e], e, (double)l[best], best)))
                    best = e;
            if (best < 0) { bad = 1; best = 0; }
            taken[best] = 1;
            topk_idx[(size_t)t * k + j] = best;
        }
        /* gates: softmax over the k chosen logits (shifted by the largest) */
        double l0 = (double)l[topk_idx[(size_t)t * k]];
        double den = 0.0;
        for (int j = 0; j < k; ++j) den += exp((double)l[topk_idx[(size_t)t * k + j]] - l0);
        for (int j = 0; j < k; ++j)
            gates[(size_t)t * k + j] = exp((double)l[topk_idx[(size_t)t * k + j]] - l0) / den;
        free(eligible);
        free(taken);
    }
    return bad ? -1 : 0;
}

/*
 * Expert co-activation counts (Cobalt page, English abstract: two experts
 * are co-activated when one token activates both). Reading: a full E x E
 * matrix where coact[a][b] counts the tokens that selected both a and b,
 * a != b; both orders are stored and the diagonal stays zero. Fresh count.
 */
int orc_coact(const int32_t* topk_idx, int T, int E, int k, int64_t* coact)
{
    if (T < 0 || E < 1 || k < 1) return -1;
    memset(coact, 0, sizeof(int64_t) * (size_t)E * (size_t)E);
    for (int t = 0; t < T; ++t)
        for (int i = 0; i < k; ++i)
            for (int j = 0; j < k; ++j) {
                if (i == j) continue;
                int a = topk_idx[(size_t)t * k + i], b = topk_idx[(size_t)t * k + j];
                if (a < 0 || a >= E || b < 0 || b >= E) return -1;
                coact[(size_t)a * E + b] += 1;
            }
    return 0;
}

/*
 * Dispatch layout over a placement of experts on G virtual ranks.
 * Zyphra page, English abstract: a dispatcher that sends each token to each
 * GPU once; experts are placed on GPUs.
 *  rank_mask[t]  : bit g set iff some selected expert of t sits on rank g.
 *  rank_off[G+1] : exclusive prefix of the per-rank row counts; R = rank_off[G].
 *  disp_token[R] : rank by rank, the tokens of that rank in ascending order
 *                  (one row per distinct (token, rank)).
 *  expert_off[E+1]: exclusive prefix of the per-expert slot counts.
 *  perm_row[T*k] : for slot s (experts ascending, tokens ascending within an
 *                  expert) the dispatched row that carries its token to the
 *                  expert's rank.
 *  slot_of[T*k]  : (t, j) -> its slot s.
 * Readings: slot and row orders as above (any grouping is valid; this one
 * is fixed), no capacity limit and no dropped or padded rows.
 */
int orc_layout(const int32_t* topk_idx, int T, int E, int k, const int32_t* place, int G,
               uint32_t* rank_mask, int32_t* rank_off, int32_t* disp_token,
               int32_t* expert_off, int32_t* perm_row, int32_t* slot_of)
{
    if (T < 0 || E < 1 || k < 1 || G < 1 || G > 32) return -1;
    for (int e = 0; e < E; ++e)
        if (place[e] < 0 || place[e] >= G) return -1;
    for (size_t i = 0; i < (size_t)T * k; ++i)
        if (topk_idx[i] < 0 || topk_idx[i] >= E) return -1;

    for (int t = 0; t < T; ++t) {
        uint32_t m = 0;
        for (int j = 0; j < k; ++j) m |= 1u << place[topk_idx[(size_t)t * k + j]];
        rank_mask[t] = m;
    }
    /* rows: rank-major, token-ascending; row_of[t*G+g] is the row of (t, g) */
    int32_t* row_of = (int32_t*)malloc(sizeof(int32_t) * ((size_t)T * G + 1));
    int32_t r = 0;
    for (int g = 0; g < G; ++g) {
        rank_off[g] = r;
        for (int t = 0; t < T; ++t) {
            if (rank_mask[t] >> g & 1u) {
                disp_token[r] = t;
                row_of[(size_t)t * G + g] = r;
                ++r;
            } else {
                row_of[(size_t)t * G + g] = -1;
            }
        }
    }
    rank_off[G] = r;
    /* slots: expert-major, token-ascending */
    int32_t s = 0;
    for (int e = 0; e < E; ++e) {
        expert_off[e] = s;
        for (int t = 0; t < T; ++t)
            for (int j = 0; j < k; ++j)
                if (topk_idx[(size_t)t * k + j] == e) {
                    perm_row[s] = row_of[(size_t)t * G + place[e]];
                    slot_of[(size_t)t * k + j] = s;
                    ++s;
                }
    }
    expert_off[E] = s;
    free(row_of);
    return 0;
}

/* Dispatched rows: row r is a copy of token disp_token[r]'s activation row. */
int orc_dispatch_rows(const void* x, int T, int d, int elem_bytes, const int32_t* disp_token,
                      int R, void* x_disp)
{
    if (d < 1 || (elem_bytes != 2 && elem_bytes != 4)) return -1;
    size_t row = (size_t)d * (size_t)elem_bytes;
    for (int i = 0; i < R; ++i) {
        if (disp_token[i] < 0 || disp_token[i] >= T) return -1;
        memcpy((char*)x_disp + (size_t)i * row, (const char*)x + (size_t)disp_token[i] * row, row);
    }
    return 0;
}

/*
 * Expert FFN on a list of rows. Reading (the pages only say "expert
 * networks"): a SwiGLU MLP without biases,
 *     u = W_gate[e] a,  v = W_up[e] a,  h = silu(u) * v,  y = W_down[e] h,
 * with silu(u) = u / (1 + exp(-u)), W_gate / W_up stored [E][F][d] and
 * W_down stored [E][d][F] (output index first).
 * Row i uses activation row src_row[i] of x ([*, d]) and expert expert[i];
 * y_out[i] gets d doubles, h_out[i] (optional) F doubles.
 */
int orc_ffn_rows(const void* x, int dt, int d, int F, int n_rows,
                 const int32_t* src_row, const int32_t* expert, int E,
                 const void* w_gate, const void* w_up, const void* w_down,
                 double* y_out, double* h_out)
{
    if (d < 1 || F < 1 || n_rows < 0 || (dt != ORC_F32 && dt != ORC_BF16)) return -1;
    for (int i = 0; i < n_rows; ++i)
        if (expert[i] < 0 || expert[i] >= E || src_row[i] < 0) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < n_rows; ++i) {
        size_t e = (size_t)expert[i];
        size_t xo = (size_t)src_row[i] * (size_t)d;
        double* a = (double*)malloc(sizeof(double) * (size_t)d);
        double* h = (double*)malloc(sizeof(double) * (size_t)F);
        for (int c = 0; c < d; ++c) a[c] = orc_elem(x, xo + (size_t)c, dt);
        for (int f = 0; f < F; ++f) {
            size_t wo = (e * (size_t)F + (size_t)f) * (size_t)d;
            double u = 0.0, v = 0.0;
            for (int c = 0; c < d; ++c) {
                u += orc_elem(w_gate, wo + (size_t)c, dt) * a[c];
                v += orc_elem(w_up, wo + (size_t)c, dt) * a[c];
            }
            h[f] = u / (1.0 + exp(-u)) * v;
        }
        for (int n = 0; n < d; ++n) {
            size_t wo = (e * (size_t)d + (size_t)n) * (size_t)F;
            double acc = 0.0;
            for (int f = 0; f < F; ++f) acc += orc_elem(w_down, wo + (size_t)f, dt) * h[f];
            y_out[(size_t)i * d + n] = acc;
        }
        if (h_out) memcpy(h_out + (size_t)i * F, h, sizeof(double) * (size_t)F);
        free(a);
        free(h);
    }
    return 0;
}

/*
 * Combine back to token order (Zyphra page, English abstract: the results
 * are combined after the experts). Reading: the gate multiplies the expert
 * output,  out[t] = sum_j gates[t][j] * y[slot_of[t*k+j]]. A negative slot
 * is a choice the replica-aware assignment dropped (Cobalt page, English
 * abstract: tokens go to expert replicas; a choice whose expert has no copy
 * has no expert output), so its term is absent.
 */
int orc_combine(const double* y, int n_slots, const int32_t* slot_of, const double* gates,
                int T, int k, int d, double* out)
{
    if (T < 0 || k < 1 || d < 1) return -1;
    for (size_t i = 0; i < (size_t)T * k; ++i)
        if (slot_of[i] >= n_slots) return -1;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                int32_t s = slot_of[(size_t)t * k + j];
                if (s < 0) continue; /* dropped choice: no expert output */
                acc += gates[(size_t)t * k + j] * y[(size_t)s * d + c];
            }
            out[(size_t)t * d + c] = acc;
        }
    }
    return 0;
}
