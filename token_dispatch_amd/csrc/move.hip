// Data-move kernels for gfx950 driven by a plan: dispatch, combine, replicate
// and the duplicate-gradient reduce. All four are HBM-bound row moves: rows are
// moved as 16-byte vectors, one wave covers 64 x 16 B = 1 KiB per instruction,
// so every global access is a fully coalesced, 1 KiB-aligned-in-row burst.
//
// Read/write phasing. On MI355X a stream of reads with a few percent of writes
// mixed in (or the reverse) runs far below either pure stream: the memory side
// pays for every switch of direction, whichever CUs or XCDs issue the minority
// traffic. Dispatch (94% writes) and combine (94% reads) therefore run as a
// short sequence of launches over token chunks, so the minority traffic of a
// chunk arrives in one burst instead of being spread over the whole kernel:
//
// dispatch  tokens are written straight into the static expert-grouped buffer
//           (news.hamidun.com EN, "Why this matters to engineers"). Each launch
//           is one resident grid; every wave first loads TPW row segments
//           (non-temporal: each is read once) into registers, then stores each
//           to the token's K slots. The reads of a chunk thus all happen at the
//           start of its launch and the rest of the launch only writes.
// combine   the weighted sum of a token's K expert outputs: one wave per
//           (token, row segment), binary32 fma in ascending k, one store; a
//           launch covers a chunk of tokens whose output is a few tens of MB.
//           Loads and stores are non-temporal (the expert outputs are read once,
//           the result is not re-read by this kernel).
// replicate duplicate experts are fetched from home before compute ("How MoonEP
//           works", same page): a fixed grid walks (duplicate slot, block piece).
// reduce    duplicate gradients back to home ("How MoonEP works"): a fixed grid
//           walks (expert with duplicates, block piece); each element is summed
//           home first, then duplicates in ascending rank.
#include "internal.h"
#include "rows.h"

namespace moonep {
namespace {

using namespace rows;

// ---------------------------------------------------------------- dispatch
// Work item = (token, segment of 64*CPL chunks). C = 16-byte chunks per row.
// One launch covers items [i_lo, i_hi); wave w of the grid takes items
// i_lo + t * n_waves + w for t < TPW, loads all of them, then stores them.
template <int CPL, int TPW>
__global__ __launch_bounds__(kMoveThreads) void k_dispatch(const v4u *__restrict__ hidden,
                                                           v4u *__restrict__ recv,
                                                           const int32_t *__restrict__ dst,
                                                           int64_t i_lo, int64_t i_hi,
                                                           int32_t segs, int32_t C, int32_t K,
                                                           int64_t n_slots) {
    const int lane = lane_id();
    const int64_t n_waves = (int64_t)gridDim.x * kMoveWaves;
    const int64_t wave = (int64_t)blockIdx.x * kMoveWaves + (threadIdx.x >> 6);
    v4u v[TPW][CPL];
    int my_dst[TPW], cbase[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int64_t item = i_lo + t * n_waves + wave;
        my_dst[t] = -1;
        cbase[t] = C;  // no chunk of an absent item passes the c < C tests
        if (item < i_hi) {
            const int64_t tok = item / segs;
            const int seg = (int)(item - tok * segs);
            cbase[t] = seg * 64 * CPL + lane;
            if (lane < K) my_dst[t] = dst[tok * K + lane];
            const v4u *row = hidden + tok * C;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = cbase[t] + i * 64;
                if (c < C) v[t][i] = __builtin_nontemporal_load(row + c);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        for (int k = 0; k < K; ++k) {
            const int d = readlane_i(my_dst[t], k);
            if (d < 0 || d >= n_slots) continue;
            v4u *out = recv + (int64_t)d * C;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = cbase[t] + i * 64;
                if (c < C) out[c] = v[t][i];
            }
        }
    }
}

// ---------------------------------------------------------------- combine
// acc += w[k] * y[dst(k)] over k ascending for one row segment (binary32 fma),
// rows read through a buffer resource (BUF) or with global loads.
template <int CPL, bool IN_BF16, bool BUF>
__device__ __forceinline__ void combine_rows(const v4u *__restrict__ y, int my_dst, float my_w,
                                             int cbase, int32_t C, int32_t K, int64_t n_slots,
                                             float (&acc)[CPL][Chunk<IN_BF16>::N]) {
    using Ch = Chunk<IN_BF16>;
    constexpr int N = Ch::N;
    for (int k = 0; k < K; ++k) {
        const int d = readlane_i(my_dst, k);
        const float wk = readlane_f(my_w, k);
        if (d < 0 || d >= n_slots) continue;
        const v4u *row = y + (int64_t)d * C;
        v4u v[CPL];
        if constexpr (BUF) {
            const __amdgpu_buffer_rsrc_t rs = row_rsrc(row, C);
#pragma unroll
            for (int i = 0; i < CPL; ++i) v[i] = load_chunk_nt(rs, cbase + i * 64);
        } else {
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = cbase + i * 64;
                v[i] = c < C ? __builtin_nontemporal_load(row + c) : v4u{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            float x[N];
            Ch::unpack(v[i], x);
#pragma unroll
            for (int j = 0; j < N; ++j) acc[i][j] = __builtin_fmaf(wk, x[j], acc[i][j]);
        }
    }
}

// One wave per work item (token, row segment) of the launch's range [i_lo, i_hi).
// Rows of at most 4 chunks per lane are held to 64 VGPRs (8 waves per SIMD, 61
// without spills instead of 71 and 7 waves): uniform's 4 KiB rows then take 4
// launches per call instead of 5, and dispatch + combine went from 0.443 to
// 0.437 ms there (one process, same buffers).
// UNIT_W: every weight is 1 and w is not read; fma(1, x, acc) is the binary32
// sum acc + x, which makes this the backward of dispatch. Rows are read through
// a buffer resource when they are shorter than about 2^31 bytes (5.26 -> 5.19 ms
// at K3, from the address arithmetic it saves), else with global loads.
template <int CPL, bool IN_BF16, bool OUT_BF16, bool UNIT_W>
__global__ __launch_bounds__(kMoveThreads) __attribute__((amdgpu_waves_per_eu(CPL <= 4 ? 8 : 1)))
void k_combine(const v4u *__restrict__ y, const float *__restrict__ w,
               const int32_t *__restrict__ dst, void *__restrict__ out, int64_t i_lo,
               int64_t i_hi, int32_t segs, int32_t C, int32_t K, int64_t n_slots) {
    using Ch = Chunk<IN_BF16>;
    constexpr int N = Ch::N;
    const int lane = lane_id();
    const int64_t item = i_lo + (int64_t)blockIdx.x * kMoveWaves + (threadIdx.x >> 6);
    if (item >= i_hi) return;
    const int64_t tok = item / segs;
    const int seg = (int)(item - tok * segs);
    const int cbase = seg * 64 * CPL + lane;
    const int my_dst = lane < K ? dst[tok * K + lane] : -1;
    const float my_w = UNIT_W ? 1.0f : (lane < K ? w[tok * K + lane] : 0.0f);

    float acc[CPL][N];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int j = 0; j < N; ++j) acc[i][j] = 0.0f;

    // the choice of load is made once per wave, outside the k loop
    if (C <= kBufRowChunks)
        combine_rows<CPL, IN_BF16, true>(y, my_dst, my_w, cbase, C, K, n_slots, acc);
    else
        combine_rows<CPL, IN_BF16, false>(y, my_dst, my_w, cbase, C, K, n_slots, acc);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = cbase + i * 64;
        if (c < C) store_elems<N, OUT_BF16, true>(out, (tok * C + c) * N, acc[i]);
    }
}

// ---------------------------------------------------------------- replicate
constexpr int kCopyUnroll = 8;                         // 16-byte chunks per thread per item
constexpr int kCopyChunks = kMoveThreads * kCopyUnroll;  // 32 KiB per work item

__global__ __launch_bounds__(kMoveThreads) void k_replicate(
    const v4u *__restrict__ expert_w, v4u *__restrict__ dup_w,
    const int32_t *__restrict__ mat_pre, const int32_t *__restrict__ dup_expert, int32_t R,
    int32_t E, int32_t B, int32_t dcap, int64_t block_chunks, int64_t items_per_slot) {
    const int64_t total = (int64_t)mat_pre[R] * items_per_slot;
    for (int64_t item = blockIdx.x; item < total; item += gridDim.x) {
        const int64_t q = item / items_per_slot;
        const int64_t part = item - q * items_per_slot;
        int lo = 0, hi = R + 1;  // rank r with mat_pre[r] <= q < mat_pre[r+1]
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (mat_pre[mid] <= q) lo = mid + 1; else hi = mid;
        }
        const int r = lo - 1;
        const int b = (int)(q - mat_pre[r]);
        const int e = dup_expert[(int64_t)r * dcap + b];
        if (e < 0 || e >= E) continue;  // only a broken plan gets here
        const v4u *s = expert_w + (int64_t)e * block_chunks;
        v4u *d = dup_w + ((int64_t)r * B + b) * block_chunks;
        const int64_t c0 = part * kCopyChunks + threadIdx.x;
        v4u v[kCopyUnroll];
#pragma unroll
        for (int i = 0; i < kCopyUnroll; ++i) {
            const int64_t c = c0 + (int64_t)i * kMoveThreads;
            if (c < block_chunks) v[i] = s[c];
        }
#pragma unroll
        for (int i = 0; i < kCopyUnroll; ++i) {
            const int64_t c = c0 + (int64_t)i * kMoveThreads;
            if (c < block_chunks) __builtin_nontemporal_store(v[i], d + c);
        }
    }
}

// ---------------------------------------------------------------- reduce
// Every byte is touched once per call, so loads and stores are non-temporal
// (2.56 -> 2.45 ms at K3). Items of 8 vectors per thread were slower.
constexpr int kRedUnroll = 4;
constexpr int kRedVecs = kMoveThreads * kRedUnroll;  // float4 per work item

__global__ __launch_bounds__(kMoveThreads) void k_reduce(
    const float4 *__restrict__ dup_grads, float4 *__restrict__ home,
    const int32_t *__restrict__ xlist, const int32_t *__restrict__ n_x,
    const int32_t *__restrict__ dup_ptr, const int32_t *__restrict__ list_rank,
    const int32_t *__restrict__ list_b, int32_t R, int32_t B, int64_t n4,
    int64_t items_per_expert) {
    const int64_t total = (int64_t)n_x[0] * items_per_expert;
    for (int64_t item = blockIdx.x; item < total; item += gridDim.x) {
        const int64_t xi = item / items_per_expert;
        const int64_t part = item - xi * items_per_expert;
        const int e = xlist[xi];
        const int p0 = dup_ptr[e], p1 = dup_ptr[e + 1];
        bool any = false;
        for (int q = p0; q < p1; ++q) any |= list_b[q] < B;
        if (!any) continue;
        float4 *h = home + (int64_t)e * n4;
        const int64_t j0 = part * kRedVecs + threadIdx.x;
        float4 acc[kRedUnroll];
#pragma unroll
        for (int i = 0; i < kRedUnroll; ++i) {
            const int64_t j = j0 + (int64_t)i * kMoveThreads;
            if (j < n4) {
                const v4f hv = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(h) + j);
                acc[i] = make_float4(hv.x, hv.y, hv.z, hv.w);
            }
        }
        for (int q = p0; q < p1; ++q) {
            const int b = list_b[q], rk = list_rank[q];
            if (b < 0 || b >= B || rk < 0 || rk >= R) continue;
            const float4 *g = dup_grads + ((int64_t)rk * B + b) * n4;
#pragma unroll
            for (int i = 0; i < kRedUnroll; ++i) {
                const int64_t j = j0 + (int64_t)i * kMoveThreads;
                if (j < n4) {
                    const v4f tv = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(g) + j);
                    const float4 t = make_float4(tv.x, tv.y, tv.z, tv.w);
                    acc[i].x = acc[i].x + t.x;
                    acc[i].y = acc[i].y + t.y;
                    acc[i].z = acc[i].z + t.z;
                    acc[i].w = acc[i].w + t.w;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kRedUnroll; ++i) {
            const int64_t j = j0 + (int64_t)i * kMoveThreads;
            if (j < n4)
                __builtin_nontemporal_store(v4f{acc[i].x, acc[i].y, acc[i].z, acc[i].w},
                                            reinterpret_cast<v4f *>(h) + j);
        }
    }
}

// Grids of the fixed-size kernels, in workgroups per CU of the 256. Replicate
// streams best with two (one process, same buffers, medians of five: K3 0.844
// against 0.890 ms with eight, decode 0.693 against 0.724, zipf 0.416 against
// 0.420), reduce with six (K3 2.314 against 2.366 ms, decode 2.022 against
// 2.081); four or fewer made reduce slower, one or three made replicate slower.
constexpr int kRepGrid = 256 * 2;
constexpr int kRedGrid = 256 * 6;

}  // namespace

thread_local int32_t *t_count_launches = nullptr;

// Dispatch launches of one resident grid each, the last one shorter. Rows of at
// most 4 chunks per lane split the items evenly over the same number of
// launches instead: a 4 KiB-row call of 1.33 resident rounds (32 768 tokens, 8
// per wave) took 0.4354 -> 0.4273 ms for dispatch + combine in one process on
// the same buffers (three runs, both orders), while wider rows were slower split
// evenly (decode 0.705 -> 0.726 ms, zipf and K3 0.3-0.7%) and keep full launches.
template <int CPL>
hipError_t dispatch_chunks(const v4u *h, v4u *r, const int32_t *dst, int64_t items, int32_t segs,
                           int32_t C, int32_t K, int64_t n_slots, hipStream_t st) {
    constexpr int TPW = tpw_of(CPL);
    static int cache[64];
    const int64_t full = resident_wgs(k_dispatch<CPL, TPW>, cache);
    int64_t per_launch = full * kMoveWaves * TPW;
    if constexpr (CPL <= 4) {  // equal launches, whole waves of TPW items each
        const int64_t n_l = (items + per_launch - 1) / per_launch;
        const int64_t q = kMoveWaves * TPW;
        per_launch = ((items + n_l - 1) / n_l + q - 1) / q * q;
    }
    for (int64_t lo = 0; lo < items; lo += per_launch) {
        const int64_t hi = items - lo < per_launch ? items : lo + per_launch;
        // the last launch only needs enough waves for what is left
        const int64_t waves = (hi - lo + TPW - 1) / TPW;
        const int64_t wgs = (waves + kMoveWaves - 1) / kMoveWaves;
        if (t_count_launches != nullptr) {
            ++*t_count_launches;
            continue;
        }
        hipLaunchKernelGGL((k_dispatch<CPL, TPW>), dim3((unsigned)(wgs < full ? wgs : full)),
                           dim3(kMoveThreads), 0, st, h, r, dst, lo, hi, segs, C, K, n_slots);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_dispatch(const PlanShape &sh, const PlanPtrs &p, const void *hidden,
                           void *recv, int64_t row_bytes, hipStream_t st) {
    const int64_t C = row_bytes / 16;
    const int cpl = pick_cpl(C);
    const int32_t segs = (int32_t)((C + 64 * cpl - 1) / (64 * cpl));
    const int64_t items = (int64_t)sh.n_tok * segs;
    const int64_t n_slots = (int64_t)sh.n_ent;
    auto h = static_cast<const v4u *>(hidden);
    auto r = static_cast<v4u *>(recv);
    switch (cpl) {
        case 1: return dispatch_chunks<1>(h, r, p.dst, items, segs, (int32_t)C, sh.K, n_slots, st);
        case 2: return dispatch_chunks<2>(h, r, p.dst, items, segs, (int32_t)C, sh.K, n_slots, st);
        case 4: return dispatch_chunks<4>(h, r, p.dst, items, segs, (int32_t)C, sh.K, n_slots, st);
        case 7: return dispatch_chunks<7>(h, r, p.dst, items, segs, (int32_t)C, sh.K, n_slots, st);
        case 8: return dispatch_chunks<8>(h, r, p.dst, items, segs, (int32_t)C, sh.K, n_slots, st);
        case 14: return dispatch_chunks<14>(h, r, p.dst, items, segs, (int32_t)C, sh.K, n_slots, st);
        case 16: return dispatch_chunks<16>(h, r, p.dst, items, segs, (int32_t)C, sh.K, n_slots, st);
        default: return hipErrorInvalidValue;
    }
}

// One combine launch is one resident round: as many items as the device holds
// waves of k_combine at once, one item per wave. Each launch's stores then come
// at the end of its reads, and the next launch's reads start after them. At K3
// that is 2048 tokens (28 MiB of output); a launch of 2048 tokens took the call
// from 5.17 ms (4096) to 5.08 ms, and half a round under-fills the device.
template <int CPL, bool IB, bool OB, bool UW>
hipError_t combine_chunks(const v4u *y, const float *w, const int32_t *dst, void *out,
                          int64_t n_tok, int32_t segs, int32_t C, int32_t K, int64_t n_slots,
                          hipStream_t st) {
    static int cache[64];
    const int64_t per_launch = (int64_t)resident_wgs(k_combine<CPL, IB, OB, UW>, cache) * kMoveWaves;
    const int64_t items = n_tok * segs;
    for (int64_t lo = 0; lo < items; lo += per_launch) {
        const int64_t hi = items - lo < per_launch ? items : lo + per_launch;
        const dim3 grid((unsigned)((hi - lo + kMoveWaves - 1) / kMoveWaves));
        if (t_count_launches != nullptr) {
            ++*t_count_launches;
            continue;
        }
        hipLaunchKernelGGL((k_combine<CPL, IB, OB, UW>), grid, dim3(kMoveThreads), 0, st, y, w, dst,
                           out, lo, hi, segs, C, K, n_slots);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <bool IB, bool OB, bool UW>
static hipError_t combine_typed(const PlanShape &sh, const PlanPtrs &p, const void *y,
                                const float *w, void *out, int64_t C, int64_t H, hipStream_t st) {
    const int cpl = pick_cpl(C);
    const int32_t segs = (int32_t)((C + 64 * cpl - 1) / (64 * cpl));
    const int64_t n_slots = (int64_t)sh.n_ent;
    auto yy = static_cast<const v4u *>(y);
#define MOONEP_COMBINE(W)                                                                  \
    case W:                                                                                \
        return combine_chunks<W, IB, OB, UW>(yy, w, p.dst, out, sh.n_tok, segs, (int32_t)C, sh.K, \
                                         n_slots, st);
    switch (cpl) {
        MOONEP_COMBINE(1)
        MOONEP_COMBINE(2)
        MOONEP_COMBINE(4)
        MOONEP_COMBINE(7)
        MOONEP_COMBINE(8)
        MOONEP_COMBINE(14)
        MOONEP_COMBINE(16)
        default: return hipErrorInvalidValue;
    }
#undef MOONEP_COMBINE
}

hipError_t launch_combine(const PlanShape &sh, const PlanPtrs &p, const void *y,
                          const float *w, void *out, int in_bf16, int out_bf16, int64_t H,
                          hipStream_t st) {
    const int64_t C = H * (in_bf16 ? 2 : 4) / 16;
    if (in_bf16 && out_bf16) return combine_typed<true, true, false>(sh, p, y, w, out, C, H, st);
    if (in_bf16) return combine_typed<true, false, false>(sh, p, y, w, out, C, H, st);
    if (out_bf16) return combine_typed<false, true, false>(sh, p, y, w, out, C, H, st);
    return combine_typed<false, false, false>(sh, p, y, w, out, C, H, st);
}

hipError_t launch_dispatch_backward(const PlanShape &sh, const PlanPtrs &p, const void *grad_recv,
                                    void *grad_hidden, int in_bf16, int out_bf16, int64_t H,
                                    hipStream_t st) {
    const int64_t C = H * (in_bf16 ? 2 : 4) / 16;
    const void *g = grad_recv;
    void *o = grad_hidden;
    if (in_bf16 && out_bf16) return combine_typed<true, true, true>(sh, p, g, nullptr, o, C, H, st);
    if (in_bf16) return combine_typed<true, false, true>(sh, p, g, nullptr, o, C, H, st);
    if (out_bf16) return combine_typed<false, true, true>(sh, p, g, nullptr, o, C, H, st);
    return combine_typed<false, false, true>(sh, p, g, nullptr, o, C, H, st);
}

hipError_t launch_replicate(const PlanShape &sh, const PlanPtrs &p, const void *expert_w,
                            void *dup_w, int64_t block_bytes, hipStream_t st) {
    if (sh.B == 0) return hipSuccess;
    const int64_t chunks = block_bytes / 16;
    const int64_t ips = (chunks + kCopyChunks - 1) / kCopyChunks;
    hipLaunchKernelGGL(k_replicate, dim3(kRepGrid), dim3(kMoveThreads), 0, st,
                       static_cast<const v4u *>(expert_w), static_cast<v4u *>(dup_w),
                       p.mat_pre, p.dup_expert, sh.R, sh.E, sh.B, sh.dcap, chunks, ips);
    return hipGetLastError();
}

hipError_t launch_reduce(const PlanShape &sh, const PlanPtrs &p, const float *dup_grads,
                         float *home_grads, int64_t block_elems, hipStream_t st) {
    if (sh.B == 0) return hipSuccess;
    const int64_t n4 = block_elems / 4;
    const int64_t ipe = (n4 + kRedVecs - 1) / kRedVecs;
    hipLaunchKernelGGL(k_reduce, dim3(kRedGrid), dim3(kMoveThreads), 0, st,
                       reinterpret_cast<const float4 *>(dup_grads),
                       reinterpret_cast<float4 *>(home_grads), p.xlist, p.n_x, p.dup_ptr,
                       p.list_rank, p.list_b, sh.R, sh.B, n4, ipe);
    return hipGetLastError();
}

}  // namespace moonep
