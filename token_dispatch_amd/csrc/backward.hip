// Backward of combine for gfx950: the gradients of the weighted sum
// out[g] = sum_k w[g,k] * y[dst(g,k)] that training needs (the layer's duplicate
// experts get gradients on the backward pass, news.hamidun.com EN, "How MoonEP
// works").
//
//   grad_w[g,k] = <grad_out[g], y[dst(g,k)]>   k_bwd_dot: pure reads (y once,
//                 grad_out once per token), one wave per token, non-temporal
//                 loads; each lane accumulates its elements with fma in eight
//                 short chains, then a fixed DPP reduction sums the 64 lanes.
//   grad_y[dst(g,k)] = w[g,k] * grad_out[g]    k_bwd_scatter: write-heavy like
//                 dispatch, so it runs the same way: resident-grid launches over
//                 token chunks, every wave first loads its grad_out row segments,
//                 then only stores the K scaled copies.
// The two run one after the other rather than fused: a fused kernel would mix
// 30 GB of reads with 30 GB of writes at the K3 shape, which MI355X serves far
// slower than the two pure-direction passes (the price is one more read of
// grad_out, 1/K of either pass).
//
// The backward of dispatch is combine with unit weights (move.hip).
#include "internal.h"
#include "rows.h"

namespace moonep {
namespace {

using namespace rows;

// v + v moved by DPP control CTRL in the rows ROWS (lanes with no source add +0).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf,
                                                          false));
}

// Sum over the 64 lanes in a fixed order; every lane gets the sum. DPP moves
// (no LDS): shifts by 1, 2, 4, 8 inside each 16-lane row, then lane 15 of a row
// into the next row and lane 31 into the upper two rows, which leaves the sum in
// lane 63.
__device__ __forceinline__ float wave_sum(float x) {
    x = dpp_add<0x111, 0xf>(x);  // row_shr:1
    x = dpp_add<0x112, 0xf>(x);  // row_shr:2
    x = dpp_add<0x114, 0xf>(x);  // row_shr:4
    x = dpp_add<0x118, 0xf>(x);  // row_shr:8
    x = dpp_add<0x142, 0xa>(x);  // row_bcast:15
    x = dpp_add<0x143, 0xc>(x);  // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// ---------------------------------------------------------------- grad_w
// One wave per token g of [t_lo, t_hi). Rows of both operands are split into
// chunks of N elements (N = 8 when both are bf16, else 4); lane l takes chunks
// l, l + 64, ... of each segment and keeps one binary32 accumulator per element
// position j of a chunk (fma in chunk order), so the eight chains are short and
// independent; they are summed j = 0..N-1, then over the lanes by a fixed
// DPP reduction. ONE_SEG: the whole grad_out row sits in registers (packed), reused
// for every k, and the y row of k+1 is loaded while k is summed.
template <bool BF16, int N>
struct RowIO;
template <>
struct RowIO<true, 8> {
    typedef v4u Raw;
    __device__ static Raw load(const void *row, int64_t c) {
        return __builtin_nontemporal_load(reinterpret_cast<const v4u *>(static_cast<const uint16_t *>(row) + c * 8));
    }
    __device__ static void unpack(const Raw &q, float *x) { Chunk<true>::unpack(q, x); }
};
template <>
struct RowIO<true, 4> {
    typedef v2u Raw;
    __device__ static Raw load(const void *row, int64_t c) {
        return __builtin_nontemporal_load(reinterpret_cast<const v2u *>(static_cast<const uint16_t *>(row) + c * 4));
    }
    __device__ static void unpack(const Raw &q, float *x) {
        x[0] = __uint_as_float(q.x << 16);
        x[1] = __uint_as_float(q.x & 0xffff0000u);
        x[2] = __uint_as_float(q.y << 16);
        x[3] = __uint_as_float(q.y & 0xffff0000u);
    }
};
template <>
struct RowIO<false, 4> {
    typedef v4u Raw;
    __device__ static Raw load(const void *row, int64_t c) {
        return __builtin_nontemporal_load(reinterpret_cast<const v4u *>(static_cast<const float *>(row) + c * 4));
    }
    __device__ static void unpack(const Raw &q, float *x) { Chunk<false>::unpack(q, x); }
};

template <int N>
__device__ __forceinline__ float sum_chains(const float *acc) {
    float s = acc[0];
#pragma unroll
    for (int j = 1; j < N; ++j) s += acc[j];
    return s;
}

template <int CPL, int N, bool G_BF16, bool Y_BF16, bool ONE_SEG>
__global__ __launch_bounds__(kMoveThreads) void k_bwd_dot(const void *__restrict__ grad_out,
                                                          const void *__restrict__ y,
                                                          const int32_t *__restrict__ dst,
                                                          float *__restrict__ grad_w,
                                                          int64_t t_lo, int64_t t_hi,
                                                          int32_t Cn, int32_t segs, int32_t K,
                                                          int64_t n_slots, int64_t H) {
    using GIO = RowIO<G_BF16, N>;
    using YIO = RowIO<Y_BF16, N>;
    constexpr int GB = G_BF16 ? 2 : 4, YB = Y_BF16 ? 2 : 4;
    const int lane = lane_id();
    const int64_t tok = t_lo + (int64_t)blockIdx.x * kMoveWaves + (threadIdx.x >> 6);
    if (tok >= t_hi) return;
    const int my_dst = lane < K ? dst[tok * K + lane] : -1;
    const char *grow = static_cast<const char *>(grad_out) + tok * H * GB;
    const char *ybase = static_cast<const char *>(y);
    float mine = 0.0f;  // lane k keeps grad_w[tok, k]
    if constexpr (ONE_SEG) {
        typename GIO::Raw g[CPL];  // packed, unpacked per k: keeps two waves per SIMD
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + i * 64;
            if (c < Cn) g[i] = GIO::load(grow, c);
        }
        typename YIO::Raw nxt[CPL];
        int dn = readlane_i(my_dst, 0);
        if (dn >= 0 && dn < n_slots) {
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = lane + i * 64;
                if (c < Cn) nxt[i] = YIO::load(ybase + (int64_t)dn * H * YB, c);
            }
        }
        for (int k = 0; k < K; ++k) {
            const int d = dn;
            typename YIO::Raw cur[CPL];
#pragma unroll
            for (int i = 0; i < CPL; ++i) cur[i] = nxt[i];
            if (k + 1 < K) {
                dn = readlane_i(my_dst, k + 1);
                if (dn >= 0 && dn < n_slots) {
#pragma unroll
                    for (int i = 0; i < CPL; ++i) {
                        const int c = lane + i * 64;
                        if (c < Cn) nxt[i] = YIO::load(ybase + (int64_t)dn * H * YB, c);
                    }
                }
            }
            float tot = 0.0f;
            if (d >= 0 && d < n_slots) {
                float acc[N];
#pragma unroll
                for (int j = 0; j < N; ++j) acc[j] = 0.0f;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    // an empty asm that "may change" g stops the compiler from
                    // hoisting its unpack out of the k loop (which would hold the
                    // row as binary32 and halve the waves per SIMD)
                    asm volatile("" : "+v"(g[i]));
                    const int c = lane + i * 64;
                    if (c < Cn) {
                        float x[N], gg[N];
                        YIO::unpack(cur[i], x);
                        GIO::unpack(g[i], gg);
#pragma unroll
                        for (int j = 0; j < N; ++j) acc[j] = __builtin_fmaf(gg[j], x[j], acc[j]);
                    }
                }
                tot = wave_sum(sum_chains<N>(acc));
            }
            if (lane == k) mine = tot;
        }
    } else {
        for (int k = 0; k < K; ++k) {
            const int d = readlane_i(my_dst, k);
            float tot = 0.0f;
            if (d >= 0 && d < n_slots) {
                const char *yrow = ybase + (int64_t)d * H * YB;
                float acc[N];
#pragma unroll
                for (int j = 0; j < N; ++j) acc[j] = 0.0f;
                for (int sg = 0; sg < segs; ++sg) {
#pragma unroll
                    for (int i = 0; i < CPL; ++i) {
                        const int c = sg * 64 * CPL + lane + i * 64;
                        if (c < Cn) {
                            float x[N], gg[N];
                            YIO::unpack(YIO::load(yrow, c), x);
                            GIO::unpack(GIO::load(grow, c), gg);
#pragma unroll
                            for (int j = 0; j < N; ++j) acc[j] = __builtin_fmaf(gg[j], x[j], acc[j]);
                        }
                    }
                }
                tot = wave_sum(sum_chains<N>(acc));
            }
            if (lane == k) mine = tot;
        }
    }
    if (lane < K) grad_w[tok * K + lane] = mine;
}

// ---------------------------------------------------------------- grad_y
// Work item = (token, segment of 64*CPL input chunks of 16 bytes). One launch is
// one resident grid over items [i_lo, i_hi); wave w takes items
// i_lo + t * n_waves + w for t < TPW, loads them all, then stores the K scaled
// copies of each.
template <int CPL, int TPW, bool G_BF16, bool Y_BF16>
__global__ __launch_bounds__(kMoveThreads) void k_bwd_scatter(const v4u *__restrict__ grad_out,
                                                              const float *__restrict__ w,
                                                              const int32_t *__restrict__ dst,
                                                              void *__restrict__ grad_y,
                                                              int64_t i_lo, int64_t i_hi,
                                                              int32_t segs, int32_t C, int32_t K,
                                                              int64_t n_slots) {
    using Ch = Chunk<G_BF16>;
    constexpr int N = Ch::N;
    const int lane = lane_id();
    const int64_t n_waves = (int64_t)gridDim.x * kMoveWaves;
    const int64_t wave = (int64_t)blockIdx.x * kMoveWaves + (threadIdx.x >> 6);
    v4u v[TPW][CPL];
    int my_dst[TPW], cbase[TPW];
    float my_w[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int64_t item = i_lo + t * n_waves + wave;
        my_dst[t] = -1;
        my_w[t] = 0.0f;
        cbase[t] = C;  // no chunk of an absent item passes the c < C tests
        if (item < i_hi) {
            const int64_t tok = item / segs;
            const int seg = (int)(item - tok * segs);
            cbase[t] = seg * 64 * CPL + lane;
            if (lane < K) {
                my_dst[t] = dst[tok * K + lane];
                my_w[t] = w[tok * K + lane];
            }
            const v4u *row = grad_out + tok * C;
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
            const float wk = readlane_f(my_w[t], k);
            if (d < 0 || d >= n_slots) continue;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = cbase[t] + i * 64;
                if (c < C) {
                    float x[N];
                    Ch::unpack(v[t][i], x);
#pragma unroll
                    for (int j = 0; j < N; ++j) x[j] = wk * x[j];
                    store_elems<N, Y_BF16, false>(grad_y, ((int64_t)d * C + c) * N, x);
                }
            }
        }
    }
}

template <int CPL, int N, bool GB, bool YB>
hipError_t dot_launch(const void *g, const void *y, const int32_t *dst, float *gw, int64_t n_tok,
                      int32_t Cn, int32_t K, int64_t n_slots, int64_t H, hipStream_t st) {
    const int32_t segs = (int32_t)((Cn + 64 * CPL - 1) / (64 * CPL));
    const dim3 grid((unsigned)((n_tok + kMoveWaves - 1) / kMoveWaves));
    if (segs == 1)
        hipLaunchKernelGGL((k_bwd_dot<CPL, N, GB, YB, true>), grid, dim3(kMoveThreads), 0, st, g,
                           y, dst, gw, (int64_t)0, n_tok, Cn, segs, K, n_slots, H);
    else
        hipLaunchKernelGGL((k_bwd_dot<CPL, N, GB, YB, false>), grid, dim3(kMoveThreads), 0, st,
                           g, y, dst, gw, (int64_t)0, n_tok, Cn, segs, K, n_slots, H);
    return hipGetLastError();
}

template <int N, bool GB, bool YB>
hipError_t dot_typed(const void *g, const void *y, const int32_t *dst, float *gw, int64_t n_tok,
                     int32_t K, int64_t n_slots, int64_t H, hipStream_t st) {
    const int32_t Cn = (int32_t)(H / N);
    switch (pick_cpl(Cn)) {
        case 1: return dot_launch<1, N, GB, YB>(g, y, dst, gw, n_tok, Cn, K, n_slots, H, st);
        case 2: return dot_launch<2, N, GB, YB>(g, y, dst, gw, n_tok, Cn, K, n_slots, H, st);
        case 4: return dot_launch<4, N, GB, YB>(g, y, dst, gw, n_tok, Cn, K, n_slots, H, st);
        case 7: return dot_launch<7, N, GB, YB>(g, y, dst, gw, n_tok, Cn, K, n_slots, H, st);
        case 8: return dot_launch<8, N, GB, YB>(g, y, dst, gw, n_tok, Cn, K, n_slots, H, st);
        case 14: return dot_launch<14, N, GB, YB>(g, y, dst, gw, n_tok, Cn, K, n_slots, H, st);
        case 16: return dot_launch<16, N, GB, YB>(g, y, dst, gw, n_tok, Cn, K, n_slots, H, st);
        default: return hipErrorInvalidValue;
    }
}

template <int CPL, bool GB, bool YB>
hipError_t scatter_chunks(const v4u *g, const float *w, const int32_t *dst, void *gy, int64_t items,
                          int32_t segs, int32_t C, int32_t K, int64_t n_slots, hipStream_t st) {
    constexpr int TPW = scaled_tpw_of(CPL);
    static int cache[64];
    const int64_t full = resident_wgs(k_bwd_scatter<CPL, TPW, GB, YB>, cache);
    const int64_t per_launch = full * kMoveWaves * TPW;
    for (int64_t lo = 0; lo < items; lo += per_launch) {
        const int64_t hi = items - lo < per_launch ? items : lo + per_launch;
        const int64_t waves = (hi - lo + TPW - 1) / TPW;
        const int64_t wgs = (waves + kMoveWaves - 1) / kMoveWaves;
        hipLaunchKernelGGL((k_bwd_scatter<CPL, TPW, GB, YB>),
                           dim3((unsigned)(wgs < full ? wgs : full)), dim3(kMoveThreads), 0, st, g,
                           w, dst, gy, lo, hi, segs, C, K, n_slots);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <bool GB, bool YB>
hipError_t scatter_typed(const PlanShape &sh, const PlanPtrs &p, const void *grad_out,
                         const float *w, void *grad_y, int64_t H, hipStream_t st) {
    const int64_t C = H * (GB ? 2 : 4) / 16;
    const int cpl = pick_cpl(C);
    const int32_t segs = (int32_t)((C + 64 * cpl - 1) / (64 * cpl));
    const int64_t items = (int64_t)sh.n_tok * segs;
    const int64_t n_slots = (int64_t)sh.n_ent;
    auto g = static_cast<const v4u *>(grad_out);
#define MOONEP_SCATTER(W) \
    case W: return scatter_chunks<W, GB, YB>(g, w, p.dst, grad_y, items, segs, (int32_t)C, sh.K, n_slots, st);
    switch (cpl) {
        MOONEP_SCATTER(1)
        MOONEP_SCATTER(2)
        MOONEP_SCATTER(4)
        MOONEP_SCATTER(7)
        MOONEP_SCATTER(8)
        MOONEP_SCATTER(14)
        MOONEP_SCATTER(16)
        default: return hipErrorInvalidValue;
    }
#undef MOONEP_SCATTER
}

}  // namespace

hipError_t launch_combine_backward(const PlanShape &sh, const PlanPtrs &p, const void *grad_out,
                                   int gout_bf16, const float *w, const void *y, void *grad_y,
                                   float *grad_w, int y_bf16, int64_t H, hipStream_t st) {
    const int64_t n_slots = (int64_t)sh.n_ent;
    if (grad_w != nullptr) {
        hipError_t e;
        if (gout_bf16 && y_bf16)
            e = dot_typed<8, true, true>(grad_out, y, p.dst, grad_w, sh.n_tok, sh.K, n_slots, H, st);
        else if (gout_bf16)
            e = dot_typed<4, true, false>(grad_out, y, p.dst, grad_w, sh.n_tok, sh.K, n_slots, H, st);
        else if (y_bf16)
            e = dot_typed<4, false, true>(grad_out, y, p.dst, grad_w, sh.n_tok, sh.K, n_slots, H, st);
        else
            e = dot_typed<4, false, false>(grad_out, y, p.dst, grad_w, sh.n_tok, sh.K, n_slots, H, st);
        if (e != hipSuccess) return e;
    }
    if (grad_y != nullptr) {
        if (gout_bf16 && y_bf16) return scatter_typed<true, true>(sh, p, grad_out, w, grad_y, H, st);
        if (gout_bf16) return scatter_typed<true, false>(sh, p, grad_out, w, grad_y, H, st);
        if (y_bf16) return scatter_typed<false, true>(sh, p, grad_out, w, grad_y, H, st);
        return scatter_typed<false, false>(sh, p, grad_out, w, grad_y, H, st);
    }
    return hipSuccess;
}

}  // namespace moonep
