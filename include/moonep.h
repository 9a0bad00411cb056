/*
 * moonep.h -- C ABI of the balanced expert-parallel hot path for MI355X (gfx950).
 *
 * The method (MoonEP, Moonshot AI, as described on news.hamidun.com EN,
 * "How MoonEP works"): every expert-parallel rank receives exactly S x K routed
 * (token, k) assignments whatever the routing skew, by scheduling a few
 * duplicate experts online from the current router output; duplicates are
 * fetched before the expert computation and their gradients are reduced back to
 * the home ranks on the backward pass. Tokens are written straight into static
 * buffers at positions grouped by expert, so no shape depends on the routing and
 * no call needs the host ("Why this matters to engineers", same page).
 *
 * On one GPU the R ranks are virtual: rank r's share of every [R, ...] array is
 * its slice [r], and moving a row between ranks is a copy between slices.
 *
 * Conventions shared by every call
 *   - All array arguments are DEVICE pointers owned by the caller. The library
 *     never allocates, frees or keeps a pointer after a call returns, and never
 *     synchronises with the host: every call only enqueues kernels on `stream`
 *     (a hipStream_t passed as void*; NULL is the default stream).
 *   - Every pointer must be non-NULL and 16-byte aligned.
 *   - Arrays are dense, row-major, in the shapes given below. Indices are int32.
 *   - Synchronous errors are the return value (checked on the host before any
 *     launch; nothing is enqueued on error). Errors that depend on data -- bad
 *     expert ids, more duplicates than B -- are bits in the plan's status word,
 *     written on the device; the caller reads it when it chooses to synchronise.
 *   - Calls that share a plan buffer must be ordered (same stream, or events).
 *     Calls on different plan buffers and outputs are independent.
 *   - The calls that take a plan (the moves and their backward) read only its
 *     first moonep_layout.persist_bytes bytes.
 */
#ifndef MOONEP_H
#define MOONEP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of hidden / expert-output rows. */
enum { MOONEP_F32 = 0, MOONEP_BF16 = 1 };

/* Return values. */
enum {
    MOONEP_OK = 0,
    MOONEP_ERR_DIMS = -1,   /* dims outside the supported range (see moonep_dims)      */
    MOONEP_ERR_PTR = -2,    /* NULL or not 16-byte aligned pointer                      */
    MOONEP_ERR_HIP = -3,    /* the HIP runtime refused a launch (hipGetLastError)      */
    MOONEP_ERR_SIZE = -4    /* a byte/element count argument is inconsistent           */
};

/* Bits of the plan's status word. */
enum {
    MOONEP_STATUS_BAD_ID = 1,    /* an id outside [0, E): that entry is dropped (dst = -1) */
    MOONEP_STATUS_REPEAT_ID = 2, /* one token names the same expert twice; the plan is
                                    still well defined, ties broken by (token, k)        */
    MOONEP_STATUS_OVER_B = 4     /* some rank needs more than B duplicates; the plan is
                                    complete, but only duplicates b < B have a slot in
                                    replicate / reduce                                  */
};

/*
 * Problem size of one MoE layer step (news.hamidun.com EN, "How MoonEP works":
 * S input tokens per rank, K experts per token; "Key facts about the release":
 * B = E/R for training, 3-4 for inference).
 *   R      ranks (virtual on one GPU), 1 <= R <= 1024
 *   E      experts, R <= E <= 1024, E % R == 0; expert e lives on rank e / (E/R)
 *   K      experts per token, 1 <= K <= min(E, 64)
 *   S      tokens per rank, S >= 1, R*S*K < 2^31
 *   B      duplicate-expert slots per rank (the [R, B, ...] shape of the
 *          duplicate weight and gradient buffers), B >= 0
 *   dtype  MOONEP_F32 or MOONEP_BF16: element type of hidden / recv / y / out
 *   H      hidden size; H * element size must be a multiple of 16 bytes
 */
typedef struct moonep_dims {
    int32_t R, E, K, S, B;
    int32_t dtype;
    int64_t H;
} moonep_dims;

/*
 * Layout of the plan buffer: ONE caller-allocated device buffer of `bytes`
 * bytes holding every plan array at the given byte offsets (all 256-byte
 * aligned). The sizes depend on the dims only. G = E/R, SK = S*K.
 *
 *   status      int32 [1]          MOONEP_STATUS_* bits
 *   maxT        int32 [1]          largest expert count
 *   maxvio      double [1]         maxT * E / (R*S*K) - 1, binary64 from exact integers
 *   T           int32 [E]          assignments routed to each expert
 *   hoff        int32 [E]          start of expert e in its home rank's (expert, token) list
 *   L           int32 [R]          home load: sum of T over the rank's G home experts
 *   keep        int32 [R]          min(L, SK): home rows kept on the rank
 *   O, D        int32 [R]          overflow L - keep and deficit SK - keep
 *   Opre, Dpre  int32 [R+1]        exclusive prefix sums of O and D
 *   dst         int32 [R*S*K]      slot of entry a = (r*S + s)*K + k, as rank*SK + row;
 *                                  -1 for a dropped entry
 *   src         int32 [R*S*K]      inverse: entry held by each slot, -1 if unfilled
 *   n_dup       int32 [R]          duplicates held by each rank (may exceed B)
 *   dup_expert  int32 [R, dcap]    expert of duplicate b of rank r (-1 beyond n_dup)
 *   dup_start   int32 [R, dcap]    its first row on the rank (-1 beyond n_dup)
 *   dup_count   int32 [R, dcap]    its rows (0 beyond n_dup)
 *   seg_ptr     int32 [R, G+dcap+1] row offsets of the rank's expert segments: home
 *                                  experts in id order, then duplicates; G+n_dup+1 used,
 *                                  -1 beyond
 *   seg_expert  int32 [R, G+dcap]  expert of each segment, -1 beyond
 *   n_list      int32 [1]          number of duplicates over all ranks
 *   list_expert, list_rank, list_b  int32 [pcap]  every duplicate, ordered by
 *                                  (expert, rank); -1 beyond n_list
 *   dup_ptr     int32 [E+1]        CSR of that list over experts
 * The remaining offsets are workspace of the plan kernels; callers must not
 * rely on their contents. Workspace that later calls read (ws_mat_pre, ws_xlist,
 * ws_n_x) lies below persist_bytes; scratch used only while the plan kernels run
 * (ws_tile_counts, ws_tile_status, ws_piece_js, ws_kept, ws_koff, ws_upre,
 * ws_pslot, ws_pcnt) lies in [persist_bytes, bytes).
 */
typedef struct moonep_layout {
    int64_t bytes;
    int64_t persist_bytes; /* the arrays above and the workspace later calls read lie in
                              [0, persist_bytes); [persist_bytes, bytes) is scratch that
                              only the plan call itself uses (see moonep_plan_noscratch) */
    int32_t dcap;          /* max(1, min(SK, E - G)): most duplicates one rank can hold */
    int32_t pcap;          /* E + R: room for the global duplicate list                 */
    int32_t n_tiles;       /* token tiles of the plan kernels                           */
    int32_t tile_tokens;   /* tokens per tile: 1024, 2048 or 4096 entries rounded down
                              to whole tokens (see plan_launches)                     */
    int32_t plan_launches; /* kernel launches of moonep_plan: 2 when a tile size keeps
                              n_tiles * E <= 65536 (the smallest such tile is used),
                              else 4 (the largest tile giving at least 256 tiles)     */
    int64_t status, maxT, maxvio, T, hoff, L, keep, O, D, Opre, Dpre, dst, src;
    int64_t n_dup, dup_expert, dup_start, dup_count, seg_ptr, seg_expert;
    int64_t n_list, list_expert, list_rank, list_b, dup_ptr;
    int64_t ws_tile_counts, ws_tile_status, ws_mat_pre, ws_xlist, ws_n_x, ws_piece_js;
    int64_t ws_kept, ws_koff, ws_upre, ws_pslot, ws_pcnt;
} moonep_layout;

/* Fills *out for dims. Pure host computation. Returns MOONEP_OK or
   MOONEP_ERR_DIMS / MOONEP_ERR_PTR (out == NULL). */
int moonep_plan_layout(const moonep_dims *dims, moonep_layout *out);

/*
 * moonep_plan -- the online redundant-expert plan of one step
 * (news.hamidun.com EN, "How MoonEP works" and "Why expert parallelism is
 * needed"; blog.schoergendorfer.com, "The problem MoonEP targets" for maxvio).
 *
 *   topk_ids  int32 [R, S, K] device, read only: the router's expert ids
 *   plan_buf  device buffer of moonep_plan_layout().bytes bytes, written
 *
 * Steps: expert histogram T and maxvio; home load L per rank; the water-fill:
 * each rank keeps the first min(L, S*K) of its home assignments in (expert,
 * token, k) order, the rest -- ordered by (home rank, expert, token, k) -- fills
 * the deficit slots of the ranks in rank order by prefix sums; each maximal run
 * of one expert inside a rank's received rows is one duplicate of that expert on
 * that rank. With valid ids every rank gets exactly S*K rows, grouped by expert.
 * The result depends on the ids only (B only sets MOONEP_STATUS_OVER_B) and is
 * bit-for-bit deterministic.
 *
 * moonep_plan_layout().plan_launches kernel launches: four (per-tile counts, a
 * scan of the counts over tiles, a one-workgroup solve, per-tile assignment), or
 * two for problems with few tiles (the decode shape): the per-tile counts, then
 * one launch in which every workgroup sums all tile counts, runs the same
 * deterministic solve and assigns its own tile -- the scheduling is "online with
 * near-zero overhead" (news.hamidun.com EN, "How MoonEP works"), and the launch
 * count is what a small step pays for. Both forms give the same plan bit for bit.
 * The plan buffer needs no initialisation; one plan buffer must not be used by
 * two calls that run at the same time.
 */
int moonep_plan(const moonep_dims *dims, const int32_t *topk_ids, void *plan_buf, void *stream);

/*
 * moonep_plan_ex -- moonep_plan with options, OR'd into flags:
 *   MOONEP_PLAN_BOUNDED      the plan of moonep_plan_bounded instead of the water-fill
 *   MOONEP_PLAN_FOUR_LAUNCH  the four-launch form whatever plan_launches says
 *   MOONEP_PLAN_TWO_LAUNCH   the two-launch form whatever plan_launches says (at
 *                            large shapes every workgroup then reads n_tiles * E
 *                            counts and runs the whole solve: correct but slow)
 * The results do not depend on the form. Unknown bits, or both forms at once,
 * return MOONEP_ERR_DIMS. moonep_plan is moonep_plan_ex with flags = 0 and
 * moonep_plan_bounded with flags = MOONEP_PLAN_BOUNDED.
 */
enum { MOONEP_PLAN_BOUNDED = 1, MOONEP_PLAN_FOUR_LAUNCH = 2, MOONEP_PLAN_TWO_LAUNCH = 4 };
int moonep_plan_ex(const moonep_dims *dims, const int32_t *topk_ids, void *plan_buf, int32_t flags,
                   void *stream);

/*
 * moonep_plan_bounded -- the same plan with at most B duplicates per rank where
 * the routing allows it, for inference budgets of a few duplicate slots per rank
 * (news.hamidun.com EN, "Key facts about the release": B of 3 to 4 for
 * inference; the pages do not say how the budget is met, so the method below is
 * this library's).
 *
 *   arguments, outputs and their layout as moonep_plan
 *
 * T, maxvio, L, keep, O, D and the S*K rows per rank are those of moonep_plan;
 * only which rows leave home, and where they go, differ:
 *   - an overloaded rank overflows its experts in (T descending, id) order, all
 *     but the last whole, and every expert keeps its first entries (token, k
 *     order) at home, packed in expert order from row 0;
 *   - deficit ranks are filled one at a time, in (D descending, rank) order;
 *     before a rank's B-th duplicate it takes the largest remaining overflow that
 *     fits whole (ties: lowest expert id), else a piece of the largest; its B-th
 *     and later duplicates take the smallest remaining overflow that fills the
 *     rest (ties: lowest id), else the largest whole;
 *   - a rank's duplicates are numbered in the order it takes them; the list is
 *     ordered by (expert, rank).
 * A rank that still needs more than B duplicates sets MOONEP_STATUS_OVER_B, as in
 * moonep_plan. Bit-for-bit deterministic; the moves and backward entry points
 * take its plan unchanged.
 */
int moonep_plan_bounded(const moonep_dims *dims, const int32_t *topk_ids, void *plan_buf,
                        void *stream);

/*
 * moonep_plan_noscratch -- moonep_plan (bounded = 0) or moonep_plan_bounded
 * (bounded = 1) for callers that cannot allocate device memory and cannot give
 * the plan room for its scratch: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.
 *
 *   topk_ids  as moonep_plan
 *   plan_buf  device buffer of at least moonep_plan_layout().persist_bytes bytes,
 *             written exactly as moonep_plan writes the same offsets; every later
 *             call (dispatch, replicate, combine, reduce, the backward moves) takes
 *             it as a plan buffer of the full size
 *   bounded   0 or 1 (anything else: MOONEP_ERR_DIMS)
 *
 * The plan kernels' scratch, bytes - persist_bytes of it, lives in one array of
 * MOONEP_STATIC_SCRATCH_BYTES in the library's device memory instead of the tail
 * of plan_buf. Each GPU holds its own copy of that array from the first call on
 * it until the process ends. Nothing is allocated or freed by the call.
 *   - A problem whose scratch exceeds MOONEP_STATIC_SCRATCH_BYTES returns
 *     MOONEP_ERR_SIZE before anything is enqueued. The scratch is about
 *     4 * E * n_tiles bytes (n_tiles from moonep_plan_layout): 1.9 MB at
 *     R = 32, E = 896, K = 16, S = 4096; 0.5 MB at R = 64, S = 128.
 *   - Every call on one GPU shares that GPU's array: two calls whose kernels may
 *     run at the same time on one GPU (different streams without ordering between
 *     them) race on it and give undefined plans. Calls ordered on one stream are
 *     safe; the kernels write the scratch before they read it, so the contents a
 *     previous call left behind never matter.
 *   - The first call on a GPU looks up the array's device address
 *     (hipGetSymbolAddress); a failure there returns MOONEP_ERR_HIP.
 * Results are bit-for-bit those of moonep_plan / moonep_plan_bounded.
 */
#define MOONEP_STATIC_SCRATCH_BYTES (8u << 20)
int moonep_plan_noscratch(const moonep_dims *dims, const int32_t *topk_ids, void *plan_buf,
                          int32_t bounded, void *stream);

/*
 * moonep_dispatch -- zero-copy scatter of token rows into the static,
 * expert-grouped receive buffer (news.hamidun.com EN, "Why this matters to
 * engineers": tokens written straight into positions grouped by expert).
 *
 *   plan_buf  read: dst
 *   hidden    [R, S, H] of dims->dtype, read; each row is read once
 *   recv      [R, S*K, H] of dims->dtype, written: recv[dst[a]] = hidden[a / K]
 *             byte for byte; every filled slot is written exactly once, unfilled
 *             slots (only after MOONEP_STATUS_BAD_ID) are left untouched.
 */
int moonep_dispatch(const moonep_dims *dims, const void *plan_buf, const void *hidden,
                    void *recv, void *stream);

/*
 * moonep_replicate -- fetch duplicate expert weights from home before the expert
 * computation (news.hamidun.com EN, "How MoonEP works": duplicates are prefetched).
 *
 *   expert_w     [E, block_bytes] read: each expert's weights as opaque bytes
 *   dup_w        [R, B, block_bytes] written: dup_w[r][b] = expert_w[dup_expert[r][b]]
 *                for b < min(n_dup[r], B); other slots are left untouched
 *   block_bytes  > 0, multiple of 16
 * With B == 0 there is nothing to copy: the call checks dims and block_bytes,
 * enqueues nothing, and the pointers may be NULL.
 */
int moonep_replicate(const moonep_dims *dims, const void *plan_buf, const void *expert_w,
                     void *dup_w, int64_t block_bytes, void *stream);

/*
 * moonep_combine -- weighted sum of each token's K expert outputs back into the
 * token's row (the router sends each token to K experts, news.hamidun.com EN,
 * "Why expert parallelism is needed").
 *
 *   y          [R, S*K, H] of dims->dtype, read: expert outputs in recv layout
 *   topk_w     float32 [R, S, K], read: router weights
 *   out        [R, S, H] of out_dtype, written:
 *              out[g] = sum over k = 0..K-1 of topk_w[g,k] * y[dst[g*K+k]],
 *              accumulated in binary32 from +0.0 with a fused multiply-add in
 *              ascending k, then stored (bf16: round to nearest even).
 *              Dropped entries (dst = -1) contribute nothing.
 *   out_dtype  MOONEP_F32 or MOONEP_BF16
 */
int moonep_combine(const moonep_dims *dims, const void *plan_buf, const void *y,
                   const float *topk_w, void *out, int32_t out_dtype, void *stream);

/*
 * moonep_reduce_dup_grads -- reduce duplicate-expert gradients back to the home
 * experts on the backward pass (news.hamidun.com EN, "How MoonEP works").
 *
 *   dup_grads    float32 [R, B, block_elems], read
 *   home_grads   float32 [E, block_elems], updated in place: for every expert e
 *                with duplicates, home_grads[e] = home_grads[e] + dup_1 + dup_2 ...
 *                over its duplicates b < B in ascending rank, binary32 adds in
 *                that fixed order. Experts without duplicates are not touched.
 *   block_elems  > 0, multiple of 4
 * With B == 0 there is nothing to add: the call checks dims and block_elems,
 * enqueues nothing, and the pointers may be NULL.
 */
int moonep_reduce_dup_grads(const moonep_dims *dims, const void *plan_buf,
                            const float *dup_grads, float *home_grads, int64_t block_elems,
                            void *stream);

/*
 * moonep_combine_backward -- gradients of combine for the backward pass. The
 * layer is trained, and its duplicate experts receive gradients on the backward
 * pass (news.hamidun.com EN, "How MoonEP works"); these are the adjoints of the
 * weighted sum that moonep_combine computes.
 *
 *   grad_out    [R, S, H] of gout_dtype, read: gradient of combine's output
 *   gout_dtype  MOONEP_F32 or MOONEP_BF16 (H * its size a multiple of 16 bytes)
 *   topk_w      float32 [R, S, K], read (may be NULL when grad_y is NULL)
 *   y           [R, S*K, H] of dims->dtype, read: the forward expert outputs
 *               (may be NULL when grad_w is NULL)
 *   grad_y      [R, S*K, H] of dims->dtype, written, or NULL to skip:
 *               grad_y[dst[a]] = topk_w[a] * grad_out[a / K], one binary32
 *               multiply per element, stored as dims->dtype (bf16: nearest even);
 *               slots that hold no entry are left untouched
 *   grad_w      float32 [R, S, K], written, or NULL to skip:
 *               grad_w[a] = sum over i of grad_out[a / K][i] * y[dst[a]][i],
 *               accumulated in binary32 in a fixed order (so within
 *               H * 2^-24 * sum |grad_out * y| of the exact value); 0 for a
 *               dropped entry
 * With both outputs NULL the call only checks its dims and returns MOONEP_OK.
 */
int moonep_combine_backward(const moonep_dims *dims, const void *plan_buf, const void *grad_out,
                            int32_t gout_dtype, const float *topk_w, const void *y, void *grad_y,
                            float *grad_w, void *stream);

/*
 * moonep_dispatch_backward -- gradient of dispatch: each token row was copied
 * to its K slots ("Why this matters to engineers", news.hamidun.com EN), so its
 * gradient is the sum of the K slot gradients.
 *
 *   grad_recv    [R, S*K, H] of dims->dtype, read
 *   grad_hidden  [R, S, H] of out_dtype, written:
 *                grad_hidden[g] = sum over k = 0..K-1 of grad_recv[dst[g*K+k]],
 *                binary32 adds in ascending k from +0.0, then stored (bf16:
 *                nearest even); dropped entries contribute nothing
 *   out_dtype    MOONEP_F32 or MOONEP_BF16
 */
int moonep_dispatch_backward(const moonep_dims *dims, const void *plan_buf, const void *grad_recv,
                             void *grad_hidden, int32_t out_dtype, void *stream);

/*
 * moonep_launch_count -- how many kernel launches one call of a chunked move
 * enqueues on the current device, for profiling: per-launch durations that a
 * kernel trace reports times this count give the call's time.
 *
 *   op          MOONEP_OP_DISPATCH (moonep_dispatch) or MOONEP_OP_COMBINE
 *               (moonep_combine with out_dtype = dims->dtype)
 *   n_launches  host, written on success
 *
 * Host only, launches nothing. The count depends on the dims and on how many
 * workgroups of the move kernel the current device holds at once (read once per
 * device). Returns MOONEP_OK, MOONEP_ERR_DIMS (bad dims or op) or
 * MOONEP_ERR_PTR (n_launches == NULL).
 */
enum { MOONEP_OP_DISPATCH = 1, MOONEP_OP_COMBINE = 2 };
int moonep_launch_count(const moonep_dims *dims, int32_t op, int32_t *n_launches);

/* Text of a return value. Never NULL; the string is static. */
const char *moonep_strerror(int rc);

#ifdef __cplusplus
}
#endif

#endif /* MOONEP_H */
