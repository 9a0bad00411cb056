// Internal interface between the C-ABI layer (api.hip) and the kernel
// translation units (plan.hip, move.hip, backward.hip). Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moonep.h"

namespace moonep {

// Hard limits of the kernels (checked by the ABI layer before any launch).
constexpr int kMaxE = 1024;        // LDS histogram bins of the plan kernels
constexpr int kMaxR = 1024;        // one rank per thread in the solve kernel
constexpr int kMaxK = 64;          // one entry of a token per lane
constexpr int kTileEntries = 4096; // most entries per plan tile (rounded down to whole tokens)
constexpr int kMinTileEntries = 1024;  // fewest: one 64-entry chunk per wave of a 16-wave tile
constexpr int kTileTarget = 256;   // tiles wanted to spread the plan over the device
// The two-launch plan (k_count, then k_plan_fused) is taken when some tile size
// keeps the counts every workgroup reads (n_tiles * E) at or below this.
constexpr int kFusedMaxCounts = 1 << 16;
constexpr int kPlanThreads = 256;  // count / assign workgroup
constexpr int kSolveThreads = 1024;

// Typed device pointers into one plan buffer, resolved from the byte layout.
struct PlanPtrs {
    int32_t *status, *maxT;
    double *maxvio;
    int32_t *T, *hoff, *L, *keep, *O, *D, *Opre, *Dpre, *dst, *src;
    int32_t *n_dup, *dup_expert, *dup_start, *dup_count, *seg_ptr, *seg_expert;
    int32_t *n_list, *list_expert, *list_rank, *list_b, *dup_ptr;
    int32_t *tile_counts, *tile_status, *mat_pre, *xlist, *n_x, *piece_js;
    int32_t *kept, *koff;  // per expert: rows kept at home, their first row there
    int32_t *upre;         // [R+1] exclusive prefix over ranks of slots left empty
    int32_t *pslot, *pcnt; // [pcap] per list entry: first slot of the piece, its rows
};

// Shape constants every kernel needs, computed once on the host.
struct PlanShape {
    int32_t R, E, K, S, B, G;
    int32_t SK;           // rows per rank
    int32_t n_tok;        // R*S
    int32_t n_ent;        // R*S*K
    int32_t dcap, pcap;
    int32_t n_tiles, tile_tokens;
    int32_t tile_chunks;  // 64-entry chunks per wave of an assign tile (1 .. 4)
    int32_t id_bits;      // bits needed to tell expert ids apart (ceil log2 E, >= 1)
    float inv_k;          // 1/K rounded to nearest: token of an in-tile entry index
    int32_t launches;     // 2: k_count + k_plan_fused; 4: k_count, k_scan, solve, k_assign
};

// Typed pointers into a plan buffer; the second form takes the plan kernels'
// scratch (the layout's [persist_bytes, bytes)) from scratch_base instead.
PlanPtrs resolve(const moonep_layout &lay, void *base);
PlanPtrs resolve(const moonep_layout &lay, void *base, void *scratch_base);

// While non-null on the calling thread, the chunked move launchers (dispatch,
// combine) add their launches to it and enqueue nothing.
extern thread_local int32_t *t_count_launches;

// bounded: the plan that keeps at most B duplicates per rank where it can
// (k_solve_bounded) instead of the water-fill (k_solve).
hipError_t launch_plan(const PlanShape &sh, const int32_t *ids, const PlanPtrs &p, bool bounded,
                       hipStream_t st);

hipError_t launch_dispatch(const PlanShape &sh, const PlanPtrs &p, const void *hidden,
                           void *recv, int64_t row_bytes, hipStream_t st);

hipError_t launch_combine(const PlanShape &sh, const PlanPtrs &p, const void *y,
                          const float *w, void *out, int in_bf16, int out_bf16, int64_t H,
                          hipStream_t st);

// The backward of dispatch: combine with unit weights (move.hip).
hipError_t launch_dispatch_backward(const PlanShape &sh, const PlanPtrs &p, const void *grad_recv,
                                    void *grad_hidden, int in_bf16, int out_bf16, int64_t H,
                                    hipStream_t st);

// The backward of combine (backward.hip): grad_w first (skipped when NULL), then
// grad_y (skipped when NULL).
hipError_t launch_combine_backward(const PlanShape &sh, const PlanPtrs &p, const void *grad_out,
                                   int gout_bf16, const float *w, const void *y, void *grad_y,
                                   float *grad_w, int y_bf16, int64_t H, hipStream_t st);

hipError_t launch_replicate(const PlanShape &sh, const PlanPtrs &p, const void *expert_w,
                            void *dup_w, int64_t block_bytes, hipStream_t st);

hipError_t launch_reduce(const PlanShape &sh, const PlanPtrs &p, const float *dup_grads,
                         float *home_grads, int64_t block_elems, hipStream_t st);

}  // namespace moonep
