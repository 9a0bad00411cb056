/*
 * moonep_oracle.c -- plain, slow, obviously correct CPU oracle for the balanced
 * expert-parallel plan and the four data moves it drives.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The product path (the HIP
 * library under token_dispatch_amd/) shares no code with it and never calls it.
 *
 * What is computed, and where it is stated (MoonEP write-ups):
 *   - the skew metric maxvio = max_e(T_e / Tbar) - 1, T_e = assignments routed to
 *     expert e, Tbar = the count under perfect balance
 *     (news.hamidun.com EN, "Why expert parallelism is needed";
 *      blog.schoergendorfer.com, "The problem MoonEP targets");
 *   - every rank receives exactly S x K assignments whatever the skew, reached by
 *     scheduling a few duplicate experts online from the current router output;
 *     duplicates are fetched before compute and their gradients are reduced back
 *     to the home ranks (news.hamidun.com EN, "How MoonEP works");
 *   - tokens are written straight into static buffers at positions grouped by
 *     expert (news.hamidun.com EN, "Why this matters to engineers").
 * The pages give no algorithm beyond this. The concrete plan below is the plain
 * water-fill reading: contiguous home experts (e / (E/R)), keep the first
 * min(L_r, S*K) home assignments of each rank in (expert, token, k) order, send
 * the rest -- ordered by (home rank, expert, token, k) -- to the deficit slots of
 * the ranks in rank order; every maximal run of one expert inside a rank's
 * deficit region is one duplicate of that expert on that rank.
 *
 * Arithmetic: integers throughout the plan; maxvio in binary64 from exact
 * integers; combine accumulates in binary32 with an explicit fused multiply-add
 * in ascending k from +0.0f and rounds the accumulator to nearest-even bf16;
 * the gradient reduce adds in binary32, home value first, then duplicates in
 * ascending rank. Build with -ffp-contract=off so that no other fusion happens.
 *
 * The data moves spread their outer loop over threads with OpenMP (built with
 * -fopenmp); each output element has one writer and its own fixed order of
 * operations, so any thread count gives the same bits as one thread.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ST_BAD_ID = 1, ST_REPEAT_ID = 2, ST_OVER_B = 4 };
enum { DT_F32 = 0, DT_BF16 = 1 };

/* Caller-owned output arrays of the plan (sizes in the comments). */
typedef struct oracle_plan_out {
    int32_t *status;     /* [1] bit flags ST_*                               */
    int64_t *maxT;       /* [1] largest expert count                         */
    double  *maxvio;     /* [1] maxT*E/(R*S*K) - 1                            */
    int32_t *T;          /* [E] assignments per expert                       */
    int32_t *hoff;       /* [E] start of expert e in its home rank's list     */
    int32_t *L;          /* [R] home load                                    */
    int32_t *keep;       /* [R] min(L, S*K)                                  */
    int32_t *O;          /* [R] overflow L - keep                            */
    int32_t *D;          /* [R] deficit S*K - keep                           */
    int32_t *Opre;       /* [R+1] exclusive prefix of O                      */
    int32_t *Dpre;       /* [R+1] exclusive prefix of D                      */
    int32_t *dst;        /* [R*S*K] slot r*S*K+s of entry a, or -1           */
    int32_t *src;        /* [R*S*K] entry placed in slot, or -1              */
    int32_t *n_dup;      /* [R]                                              */
    int32_t *dup_expert; /* [R*dcap] -1 beyond n_dup                         */
    int32_t *dup_start;  /* [R*dcap] first slot of the run, -1 beyond n_dup  */
    int32_t *dup_count;  /* [R*dcap] rows of the run, 0 beyond n_dup         */
    int32_t *seg_ptr;    /* [R*(G+dcap+1)] row offsets of rank segments, -1 pad */
    int32_t *seg_expert; /* [R*(G+dcap)]   expert of each segment, -1 pad    */
    int32_t *n_list;     /* [1] number of duplicates over all ranks          */
    int32_t *list_expert;/* [pcap] duplicates ordered by (expert, rank)      */
    int32_t *list_rank;  /* [pcap]                                           */
    int32_t *list_b;     /* [pcap] index of the duplicate on its rank        */
    int32_t *dup_ptr;    /* [E+1] CSR of the list over experts               */
} oracle_plan_out;

static int64_t find_deficit_rank(const int32_t *Dpre, int R, int64_t j)
{
    /* the unique r with Dpre[r] <= j < Dpre[r+1] (a plain linear walk) */
    for (int r = 0; r < R; ++r)
        if (Dpre[r] <= j && j < Dpre[r + 1]) return r;
    return -1;
}

/* Returns 0, or -1 on inconsistent arguments. */
int oracle_plan(int32_t R, int32_t E, int32_t K, int32_t S, int32_t B,
                const int32_t *ids, int32_t dcap, int32_t pcap, oracle_plan_out *o)
{
    if (R <= 0 || E <= 0 || K <= 0 || S <= 0 || B < 0 || E % R != 0 || K > E) return -1;
    const int64_t G = E / R, SK = (int64_t)S * K, N = (int64_t)R * S, NE = N * K;
    int32_t status = 0;

    /* Step 0: validate. Entries with an id outside [0,E) take part in nothing. */
    for (int64_t g = 0; g < N; ++g)
        for (int k = 0; k < K; ++k) {
            int32_t e = ids[g * K + k];
            if (e < 0 || e >= E) { status |= ST_BAD_ID; continue; }
            for (int k2 = 0; k2 < k; ++k2)
                if (ids[g * K + k2] == e) status |= ST_REPEAT_ID;
        }

    /* Step 1: histogram and maxvio. Tbar = R*S*K / E. */
    for (int e = 0; e < E; ++e) o->T[e] = 0;
    for (int64_t a = 0; a < NE; ++a)
        if (ids[a] >= 0 && ids[a] < E) o->T[ids[a]] += 1;
    int64_t maxT = 0;
    for (int e = 0; e < E; ++e) if (o->T[e] > maxT) maxT = o->T[e];
    *o->maxT = maxT;
    *o->maxvio = (double)(maxT * (int64_t)E) / (double)NE - 1.0;

    /* Step 2: home load. Expert e lives on rank e / G. */
    for (int r = 0; r < R; ++r) {
        int64_t acc = 0;
        for (int64_t i = 0; i < G; ++i) {
            o->hoff[r * G + i] = (int32_t)acc;
            acc += o->T[r * G + i];
        }
        o->L[r] = (int32_t)acc;
    }

    /* Step 3a: water-fill quantities. */
    o->Opre[0] = 0;
    o->Dpre[0] = 0;
    for (int r = 0; r < R; ++r) {
        o->keep[r] = o->L[r] < SK ? o->L[r] : (int32_t)SK;
        o->O[r] = o->L[r] - o->keep[r];
        o->D[r] = (int32_t)SK - o->keep[r];
        o->Opre[r + 1] = o->Opre[r] + o->O[r];
        o->Dpre[r + 1] = o->Dpre[r] + o->D[r];
    }

    /* Step 3b: place every entry. pos = earlier entries of the same expert. */
    for (int64_t s = 0; s < NE; ++s) o->src[s] = -1;
    int32_t *seen = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    if (!seen) return -1;
    for (int64_t a = 0; a < NE; ++a) {
        int32_t e = ids[a];
        if (e < 0 || e >= E) { o->dst[a] = -1; continue; }
        int64_t r = e / G;
        int64_t h = (int64_t)o->hoff[e] + seen[e];
        seen[e] += 1;
        int64_t d, slot;
        if (h < SK) {
            d = r;
            slot = h;
        } else {
            int64_t j = o->Opre[r] + (h - SK);
            d = find_deficit_rank(o->Dpre, R, j);
            if (d < 0) { free(seen); return -1; }  /* Opre[R] != Dpre[R]: inconsistent */
            slot = o->keep[d] + (j - o->Dpre[d]);
        }
        if (slot < 0 || slot >= SK) { free(seen); return -1; }
        o->dst[a] = (int32_t)(d * SK + slot);
        o->src[d * SK + slot] = (int32_t)a;
    }
    free(seen);

    /* Step 3c: duplicates = maximal runs of one expert among the slots a rank
       received beyond its kept rows. Unfilled slots (src == -1) end the walk. */
    for (int64_t i = 0; i < (int64_t)R * dcap; ++i) {
        o->dup_expert[i] = -1;
        o->dup_start[i] = -1;
        o->dup_count[i] = 0;
    }
    for (int r = 0; r < R; ++r) {
        int32_t nd = 0;
        int64_t s = o->keep[r];
        while (s < SK && o->src[r * SK + s] >= 0) {
            int32_t e = ids[o->src[r * SK + s]];
            int64_t s0 = s;
            while (s < SK && o->src[r * SK + s] >= 0 && ids[o->src[r * SK + s]] == e) ++s;
            if (nd >= dcap) return -1;
            o->dup_expert[(int64_t)r * dcap + nd] = e;
            o->dup_start[(int64_t)r * dcap + nd] = (int32_t)s0;
            o->dup_count[(int64_t)r * dcap + nd] = (int32_t)(s - s0);
            ++nd;
        }
        o->n_dup[r] = nd;
        if (nd > B) status |= ST_OVER_B;
    }

    /* Step 3d: per-rank segments: home experts in id order, then duplicates. */
    const int64_t sp = G + dcap + 1, se = G + dcap;
    for (int r = 0; r < R; ++r) {
        for (int64_t i = 0; i < sp; ++i) o->seg_ptr[r * sp + i] = -1;
        for (int64_t i = 0; i < se; ++i) o->seg_expert[r * se + i] = -1;
        for (int64_t i = 0; i < G; ++i) {
            int64_t st = o->hoff[r * G + i];
            o->seg_ptr[r * sp + i] = (int32_t)(st < SK ? st : SK);
            o->seg_expert[r * se + i] = (int32_t)(r * G + i);
        }
        int64_t end = o->keep[r];
        for (int b = 0; b < o->n_dup[r]; ++b) {
            o->seg_ptr[r * sp + G + b] = o->dup_start[(int64_t)r * dcap + b];
            o->seg_expert[r * se + G + b] = o->dup_expert[(int64_t)r * dcap + b];
            end = o->dup_start[(int64_t)r * dcap + b] + o->dup_count[(int64_t)r * dcap + b];
        }
        o->seg_ptr[r * sp + G + o->n_dup[r]] = (int32_t)end;
    }

    /* Step 3e: all duplicates ordered by (expert, rank), CSR over experts. */
    for (int32_t p = 0; p < pcap; ++p) {
        o->list_expert[p] = -1;
        o->list_rank[p] = -1;
        o->list_b[p] = -1;
    }
    int32_t p = 0;
    for (int e = 0; e < E; ++e) {
        o->dup_ptr[e] = p;
        for (int r = 0; r < R; ++r)
            for (int b = 0; b < o->n_dup[r]; ++b)
                if (o->dup_expert[(int64_t)r * dcap + b] == e) {
                    if (p >= pcap) return -1;
                    o->list_expert[p] = e;
                    o->list_rank[p] = r;
                    o->list_b[p] = b;
                    ++p;
                }
    }
    o->dup_ptr[E] = p;
    *o->n_list = p;
    *o->status = status;
    return 0;
}

/* Dispatch: recv[slot] = hidden[token of the entry placed there], byte for
   byte. Only slots in [slot_lo, slot_hi) are written, into recv_window, whose
   row 0 is slot slot_lo (this lets a caller stream the output by rank). */
void oracle_dispatch(int64_t n_ent, int32_t K, int64_t row_bytes, const uint8_t *hidden,
                     const int32_t *dst, int64_t slot_lo, int64_t slot_hi, uint8_t *recv_window)
{
    #pragma omp parallel for schedule(static)
    for (int64_t a = 0; a < n_ent; ++a) {
        int64_t d = dst[a];
        if (d < slot_lo || d >= slot_hi) continue;
        memcpy(recv_window + (d - slot_lo) * row_bytes, hidden + (a / K) * row_bytes,
               (size_t)row_bytes);
    }
}

/* Replicate: dup_w[r][b] = expert_w[dup_expert[r][b]] for b < min(n_dup[r], B). */
void oracle_replicate(int32_t R, int32_t B, int32_t dcap, const int32_t *n_dup,
                      const int32_t *dup_expert, int64_t block_bytes,
                      const uint8_t *expert_w, uint8_t *dup_w)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < R; ++r)
        for (int b = 0; b < n_dup[r] && b < B; ++b)
            memcpy(dup_w + ((int64_t)r * B + b) * block_bytes,
                   expert_w + (int64_t)dup_expert[(int64_t)r * dcap + b] * block_bytes,
                   (size_t)block_bytes);
}

static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round binary32 to the nearest bf16, ties to even; NaN stays a quiet NaN. */
static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* Combine: out[g] = sum_k w[g,k] * y[dst[g,k]], fp32 accumulation from +0.0f in
   ascending k with fmaf, then stored as out_dtype. Entries with dst < 0 are
   skipped. Tokens g in [0, n_tok). */
void oracle_combine(int64_t n_tok, int32_t K, int64_t H, int32_t in_dtype, int32_t out_dtype,
                    const void *y, const int32_t *dst, const float *w, void *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < n_tok; ++g)
        for (int64_t i = 0; i < H; ++i) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                int64_t d = dst[g * K + k];
                if (d < 0) continue;
                float x = in_dtype == DT_BF16 ? bf16_to_f32(((const uint16_t *)y)[d * H + i])
                                              : ((const float *)y)[d * H + i];
                acc = fmaf(w[g * K + k], x, acc);
            }
            if (out_dtype == DT_BF16)
                ((uint16_t *)out)[g * H + i] = f32_to_bf16_rne(acc);
            else
                ((float *)out)[g * H + i] = acc;
        }
}

/* Reduce: for each expert e, home[e] = home[e] + dup_1 + dup_2 + ... over its
   duplicates in list order (ascending rank), skipping duplicates with b >= B,
   which have no slot. dup_grads is [R, B, n], home is [E, n], updated in place. */
void oracle_reduce(int32_t E, int32_t B, int64_t n, const int32_t *dup_ptr,
                   const int32_t *list_rank, const int32_t *list_b,
                   const float *dup_grads, float *home)
{
    #pragma omp parallel for collapse(2) schedule(static)
    for (int e = 0; e < E; ++e)
        for (int64_t i = 0; i < n; ++i) {
            float v = home[(int64_t)e * n + i];
            for (int32_t p = dup_ptr[e]; p < dup_ptr[e + 1]; ++p) {
                if (list_b[p] >= B) continue;
                v = v + dup_grads[((int64_t)list_rank[p] * B + list_b[p]) * n + i];
            }
            home[(int64_t)e * n + i] = v;
        }
}

/* Threads of the data moves and their backward (the plan is one thread: its
   prefix sums and running counters are sequential). Every output element of a
   move has exactly one writer -- a slot holds one entry, a token row, an expert
   element -- so the results do not depend on the number of threads. */
void oracle_set_threads(int32_t n) { omp_set_num_threads(n > 0 ? n : 1); }
int32_t oracle_max_threads(void) { return (int32_t)omp_get_max_threads(); }

/* The rounding used by combine, exposed so tests can pin it to a library. */
void oracle_f32_to_bf16(int64_t n, const float *x, uint16_t *y)
{
    for (int64_t i = 0; i < n; ++i) y[i] = f32_to_bf16_rne(x[i]);
}

/* ---------------------------------------------------------------- backward
 * The forward moves are linear maps, and training (the pages speak of gradients
 * reduced back to home on the backward pass, news.hamidun.com EN, "How MoonEP
 * works") needs their adjoints:
 *   combine  out[g] = sum_k w[g,k] * y[dst(g,k)]
 *     grad_y[dst(g,k)] = w[g,k] * grad_out[g]          (one binary32 multiply,
 *                                                      stored in y's type)
 *     grad_w[g,k]      = sum_i grad_out[g][i] * y[dst(g,k)][i]   (binary64 here)
 *   dispatch recv[dst(a)] = hidden[a / K]
 *     grad_hidden[g]   = sum_k grad_recv[dst(g,k)]      (binary32 adds in
 *                                                      ascending k from +0.0)
 * Entries with dst < 0 contribute nothing; their grad_w is 0.
 */
static float load_elem(const void *base, int32_t dtype, int64_t idx)
{
    return dtype == DT_BF16 ? bf16_to_f32(((const uint16_t *)base)[idx]) : ((const float *)base)[idx];
}

static void store_elem(void *base, int32_t dtype, int64_t idx, float v)
{
    if (dtype == DT_BF16) ((uint16_t *)base)[idx] = f32_to_bf16_rne(v);
    else ((float *)base)[idx] = v;
}

/* grad_y rows for slots [slot_lo, slot_hi) into grad_y_window (row 0 = slot_lo).
   Slots that hold no entry are not written. */
void oracle_combine_backward_y(int64_t n_ent, int32_t K, int64_t H, int32_t gout_dtype,
                               int32_t y_dtype, const void *grad_out, const float *w,
                               const int32_t *dst, int64_t slot_lo, int64_t slot_hi,
                               void *grad_y_window)
{
    #pragma omp parallel for schedule(static)
    for (int64_t a = 0; a < n_ent; ++a) {
        int64_t d = dst[a];
        if (d < slot_lo || d >= slot_hi) continue;
        int64_t g = a / K;
        for (int64_t i = 0; i < H; ++i) {
            float x = load_elem(grad_out, gout_dtype, g * H + i);
            float v = w[a] * x;
            store_elem(grad_y_window, y_dtype, (d - slot_lo) * H + i, v);
        }
    }
}

/* grad_w[a] for tokens g in [0, n_tok), a = g*K + k, in binary64. y_rows holds the
   expert-output row of every entry: y_rows[a] = y[dst(a)] (a caller may gather
   just the rows it samples); entries with dst < 0 give 0. */
void oracle_combine_backward_w(int64_t n_tok, int32_t K, int64_t H, int32_t gout_dtype,
                               int32_t y_dtype, const void *grad_out, const void *y_rows,
                               const int32_t *dst, double *grad_w)
{
    #pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < n_tok; ++g)
        for (int k = 0; k < K; ++k) {
            int64_t a = g * K + k;
            double s = 0.0;
            if (dst[a] >= 0)
                for (int64_t i = 0; i < H; ++i)
                    s += (double)load_elem(grad_out, gout_dtype, g * H + i) *
                         (double)load_elem(y_rows, y_dtype, a * H + i);
            grad_w[a] = s;
        }
}

/* grad_hidden[g] = sum over k of grad_recv[dst(g,k)], binary32 adds in ascending k
   from +0.0, stored as out_dtype. */
void oracle_dispatch_backward(int64_t n_tok, int32_t K, int64_t H, int32_t in_dtype,
                              int32_t out_dtype, const void *grad_recv, const int32_t *dst,
                              void *grad_hidden)
{
    #pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < n_tok; ++g)
        for (int64_t i = 0; i < H; ++i) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                int64_t d = dst[g * K + k];
                if (d < 0) continue;
                acc = acc + load_elem(grad_recv, in_dtype, d * H + i);
            }
            store_elem(grad_hidden, out_dtype, g * H + i, acc);
        }
}

/* ---------------------------------------------------------------- bounded plan
 * A plan for inference, where each rank should hold at most B duplicate experts
 * (news.hamidun.com EN, "Key facts about the release": B = 3-4 for inference).
 * The pages do not say how the bound is met; this is the reading used here. It
 * keeps exact S*K rows per rank and the same (minimum) number of moved rows as
 * the water-fill, and changes two choices:
 *   1. which home rows overflow: an overloaded rank overflows its largest
 *      experts first (home experts ordered by T descending, then id), so the
 *      same O_r rows leave through as few experts as possible; inside an expert
 *      the kept rows are its first (token, k) entries and the overflow its last;
 *   2. where the overflow goes: deficit ranks are filled one at a time, in order
 *      of deficit D descending (then rank id); a rank's pieces 1 .. B-1 are whole
 *      items -- the largest remaining overflow that fits (then lowest expert id),
 *      or, if none fits, a piece of the largest remaining overflow that fills the
 *      rank; its B-th piece is a piece of the smallest remaining overflow that is
 *      at least the rank's free room (then lowest expert id), which fills it, or
 *      if no overflow is that large, the largest remaining one whole. A rank
 *      that still has room after B pieces goes on the same way and
 *      ST_OVER_B is raised.
 * Rows of a rank: home experts in id order (kept rows only), then its pieces in
 * the order they were placed. Every other table has the water-fill's meaning.
 */
int oracle_plan_bounded(int32_t R, int32_t E, int32_t K, int32_t S, int32_t B,
                        const int32_t *ids, int32_t dcap, int32_t pcap, oracle_plan_out *o)
{
    if (R <= 0 || E <= 0 || K <= 0 || S <= 0 || B < 0 || E % R != 0 || K > E) return -1;
    const int64_t G = E / R, SK = (int64_t)S * K, N = (int64_t)R * S, NE = N * K;
    int32_t status = 0;

    /* validate, histogram, maxvio, home offsets and the water-fill quantities:
       exactly as in oracle_plan */
    for (int64_t g = 0; g < N; ++g)
        for (int k = 0; k < K; ++k) {
            int32_t e = ids[g * K + k];
            if (e < 0 || e >= E) { status |= ST_BAD_ID; continue; }
            for (int k2 = 0; k2 < k; ++k2)
                if (ids[g * K + k2] == e) status |= ST_REPEAT_ID;
        }
    for (int e = 0; e < E; ++e) o->T[e] = 0;
    for (int64_t a = 0; a < NE; ++a)
        if (ids[a] >= 0 && ids[a] < E) o->T[ids[a]] += 1;
    int64_t maxT = 0;
    for (int e = 0; e < E; ++e) if (o->T[e] > maxT) maxT = o->T[e];
    *o->maxT = maxT;
    *o->maxvio = (double)(maxT * (int64_t)E) / (double)NE - 1.0;
    for (int r = 0; r < R; ++r) {
        int64_t acc = 0;
        for (int64_t i = 0; i < G; ++i) {
            o->hoff[r * G + i] = (int32_t)acc;
            acc += o->T[r * G + i];
        }
        o->L[r] = (int32_t)acc;
    }
    o->Opre[0] = 0;
    o->Dpre[0] = 0;
    for (int r = 0; r < R; ++r) {
        o->keep[r] = o->L[r] < SK ? o->L[r] : (int32_t)SK;
        o->O[r] = o->L[r] - o->keep[r];
        o->D[r] = (int32_t)SK - o->keep[r];
        o->Opre[r + 1] = o->Opre[r] + o->O[r];
        o->Dpre[r + 1] = o->Dpre[r] + o->D[r];
    }

    int64_t *ov = (int64_t *)calloc((size_t)E, sizeof(int64_t));    /* overflow rows   */
    int64_t *left = (int64_t *)calloc((size_t)E, sizeof(int64_t));  /* not yet placed  */
    int64_t *koff = (int64_t *)calloc((size_t)E, sizeof(int64_t));  /* home slot start */
    int32_t *seen = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    int32_t *taken = (int32_t *)calloc((size_t)G, sizeof(int32_t));
    /* pieces in placement order */
    int32_t *pe = (int32_t *)malloc(sizeof(int32_t) * (size_t)(pcap > 0 ? pcap : 1));
    int32_t *pr = (int32_t *)malloc(sizeof(int32_t) * (size_t)(pcap > 0 ? pcap : 1));
    int64_t *pstart = (int64_t *)malloc(sizeof(int64_t) * (size_t)(pcap > 0 ? pcap : 1));
    int64_t *pcount = (int64_t *)malloc(sizeof(int64_t) * (size_t)(pcap > 0 ? pcap : 1));
    int64_t *pfirst = (int64_t *)malloc(sizeof(int64_t) * (size_t)(pcap > 0 ? pcap : 1));
    int32_t *rdone = (int32_t *)calloc((size_t)R, sizeof(int32_t));
    int rc = -1;
    if (!ov || !left || !koff || !seen || !taken || !pe || !pr || !pstart || !pcount || !pfirst || !rdone)
        goto out;

    /* 1. overflow of each overloaded rank, from its largest experts */
    for (int r = 0; r < R; ++r) {
        int64_t rem = o->O[r];
        for (int64_t i = 0; i < G; ++i) taken[i] = 0;
        while (rem > 0) {
            int64_t best = -1;
            for (int64_t i = 0; i < G; ++i)
                if (!taken[i] && (best < 0 || o->T[r * G + i] > o->T[r * G + best])) best = i;
            if (best < 0) goto out;
            taken[best] = 1;
            int64_t e = r * G + best;
            int64_t t = o->T[e] < rem ? o->T[e] : rem;
            ov[e] = t;
            rem -= t;
        }
        int64_t acc = 0;  /* kept rows in id order */
        for (int64_t i = 0; i < G; ++i) {
            koff[r * G + i] = acc;
            acc += o->T[r * G + i] - ov[r * G + i];
        }
    }
    for (int e = 0; e < E; ++e) left[e] = ov[e];

    /* 2. fill the deficit ranks, largest deficit first */
    int32_t np = 0;
    for (int step = 0; step < R; ++step) {
        int r = -1;
        for (int q = 0; q < R; ++q)
            if (!rdone[q] && o->D[q] > 0 && (r < 0 || o->D[q] > o->D[r])) r = q;
        if (r < 0) break;
        rdone[r] = 1;
        int64_t room = o->D[r];
        int32_t used = 0;
        while (room > 0) {
            int e = -1;
            if (used < B - 1) {
                /* largest overflow that fits whole, else the largest (split) */
                for (int x = 0; x < E; ++x)
                    if (left[x] > 0 && left[x] <= room && (e < 0 || left[x] > left[e])) e = x;
                if (e < 0)
                    for (int x = 0; x < E; ++x)
                        if (left[x] > 0 && (e < 0 || left[x] > left[e])) e = x;
            } else {
                /* smallest overflow that fills the room, else the largest */
                for (int x = 0; x < E; ++x)
                    if (left[x] >= room && (e < 0 || left[x] < left[e])) e = x;
                if (e < 0)
                    for (int x = 0; x < E; ++x)
                        if (left[x] > 0 && (e < 0 || left[x] > left[e])) e = x;
            }
            if (e < 0) break;  /* nothing left to place (only when ids were dropped) */
            if (np >= pcap) goto out;
            int64_t t = left[e] < room ? left[e] : room;
            pe[np] = e;
            pr[np] = r;
            pstart[np] = o->keep[r] + (o->D[r] - room);
            pcount[np] = t;
            pfirst[np] = ov[e] - left[e];
            ++np;
            left[e] -= t;
            room -= t;
            ++used;
        }
    }

    /* 3. place every entry: kept rows at home, overflow rows in their piece */
    for (int64_t s = 0; s < NE; ++s) o->src[s] = -1;
    for (int64_t a = 0; a < NE; ++a) {
        int32_t e = ids[a];
        if (e < 0 || e >= E) { o->dst[a] = -1; continue; }
        int64_t r = e / G, h = seen[e]++;
        int64_t kept = o->T[e] - ov[e];
        int64_t slot = -1;
        if (h < kept) {
            slot = r * SK + koff[e] + h;
        } else {
            int64_t j = h - kept;
            for (int32_t q = 0; q < np; ++q)
                if (pe[q] == e && pfirst[q] <= j && j < pfirst[q] + pcount[q])
                    slot = pr[q] * SK + pstart[q] + (j - pfirst[q]);
        }
        if (slot < 0 || slot >= NE) goto out;
        o->dst[a] = (int32_t)slot;
        o->src[slot] = (int32_t)a;
    }

    /* 4. duplicate tables (pieces of each rank in placement order), segments,
          and the global list ordered by (expert, rank) */
    for (int64_t i = 0; i < (int64_t)R * dcap; ++i) {
        o->dup_expert[i] = -1;
        o->dup_start[i] = -1;
        o->dup_count[i] = 0;
    }
    const int64_t sp = G + dcap + 1, se = G + dcap;
    for (int r = 0; r < R; ++r) {
        int32_t b = 0;
        int64_t end = o->keep[r];
        for (int64_t i = 0; i < sp; ++i) o->seg_ptr[r * sp + i] = -1;
        for (int64_t i = 0; i < se; ++i) o->seg_expert[r * se + i] = -1;
        for (int64_t i = 0; i < G; ++i) {
            o->seg_ptr[r * sp + i] = (int32_t)koff[r * G + i];
            o->seg_expert[r * se + i] = (int32_t)(r * G + i);
        }
        for (int32_t q = 0; q < np; ++q) {
            if (pr[q] != r) continue;
            if (b >= dcap) goto out;
            o->dup_expert[(int64_t)r * dcap + b] = pe[q];
            o->dup_start[(int64_t)r * dcap + b] = (int32_t)pstart[q];
            o->dup_count[(int64_t)r * dcap + b] = (int32_t)pcount[q];
            o->seg_ptr[r * sp + G + b] = (int32_t)pstart[q];
            o->seg_expert[r * se + G + b] = pe[q];
            end = pstart[q] + pcount[q];
            ++b;
        }
        o->seg_ptr[r * sp + G + b] = (int32_t)end;
        o->n_dup[r] = b;
        if (b > B) status |= ST_OVER_B;
    }
    for (int32_t p = 0; p < pcap; ++p) {
        o->list_expert[p] = -1;
        o->list_rank[p] = -1;
        o->list_b[p] = -1;
    }
    int32_t p = 0;
    for (int e = 0; e < E; ++e) {
        o->dup_ptr[e] = p;
        for (int r = 0; r < R; ++r)
            for (int b = 0; b < o->n_dup[r]; ++b)
                if (o->dup_expert[(int64_t)r * dcap + b] == e) {
                    o->list_expert[p] = e;
                    o->list_rank[p] = r;
                    o->list_b[p] = b;
                    ++p;
                }
    }
    o->dup_ptr[E] = p;
    *o->n_list = p;
    *o->status = status;
    rc = 0;
out:
    free(ov); free(left); free(koff); free(seen); free(taken);
    free(pe); free(pr); free(pstart); free(pcount); free(pfirst); free(rdone);
    return rc;
}
