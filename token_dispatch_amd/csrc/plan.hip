// Plan kernels for gfx950: the online redundant-expert plan of one step.
//
// The method (news.hamidun.com EN, "How MoonEP works"): every rank receives
// exactly S*K (token, k) assignments whatever the routing skew, by scheduling a
// few duplicate experts from the current router output. Skew is measured as
// maxvio = max_e(T_e / Tbar) - 1 ("Why expert parallelism is needed", same page;
// blog.schoergendorfer.com, "The problem MoonEP targets").
//
// Four launches, every grid fixed by the dims alone (no host round trip):
//   k_count   one workgroup per token tile: validates ids, builds the tile's
//             expert histogram in LDS, writes it to tile_counts[tile][E].
//   k_scan    one workgroup per 64 experts: exclusive scan of tile_counts down
//             the tiles (in place) and the column totals T[e].
//   k_solve   one workgroup: home offsets, home load, keep / overflow / deficit
//             and their prefix sums, then the duplicates as the intersections of
//             each expert's overflow interval with each rank's deficit interval
//             (a merge of two sorted boundary lists), and all plan tables.
//   k_assign  one workgroup per token tile: the stable position of every entry
//             inside its expert (tile base + per-wave LDS base + in-wave rank from
//             bit-sliced ballots), then its slot, and the inverse map.
//
// Why this is exact: entry a's position inside expert e is the number of
// earlier entries with id e. That count is split as (earlier tiles) + (earlier
// waves of this tile) + (earlier lanes of the same 64-entry chunk) + (earlier
// chunks of this wave), each an integer count taken in entry order.
#include "internal.h"

namespace moonep {
namespace {

constexpr int kWaves = kPlanThreads / 64;

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Inclusive scan over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x;
}

__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x = max(x, __shfl_xor(x, d, 64));
    return x;
}

// Exclusive scan of one value per thread over a 1024-thread workgroup.
// s_w needs 17 ints. Every thread must call it. Returns the exclusive prefix.
__device__ int block_excl_scan(int v, int *s_w, int &total) {
    const int lane = lane_id(), w = threadIdx.x >> 6;
    const int inc = wave_incl_scan(v);
    if (lane == 63) s_w[w] = inc;
    __syncthreads();
    if (w == 0) {
        int t = lane < kSolveThreads / 64 ? s_w[lane] : 0;
        int ti = wave_incl_scan(t);
        if (lane < kSolveThreads / 64) s_w[lane] = ti - t;
        if (lane == kSolveThreads / 64 - 1) s_w[16] = ti;
    }
    __syncthreads();
    const int res = inc - v + s_w[w];
    total = s_w[16];
    __syncthreads();
    return res;
}

__device__ int block_max(int v, int *s_w) {
    const int lane = lane_id(), w = threadIdx.x >> 6;
    v = wave_max(v);
    if (lane == 0) s_w[w] = v;
    __syncthreads();
    int m = s_w[0];
    for (int i = 1; i < kSolveThreads / 64; ++i) m = max(m, s_w[i]);
    __syncthreads();
    return m;
}

// First index i in [0, n) with a[i] > x (n if none).
__device__ __forceinline__ int upper_bound(const int *a, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (a[mid] <= x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// First index i in [0, n) with a[i] >= x (n if none).
__device__ __forceinline__ int lower_bound(const int *a, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (a[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// ---------------------------------------------------------------- k_count
__global__ __launch_bounds__(kPlanThreads) void k_count(const int32_t *__restrict__ ids,
                                                        PlanShape sh,
                                                        int32_t *__restrict__ tile_counts,
                                                        int32_t *__restrict__ tile_status) {
    __shared__ int32_t s_hist[kMaxE];
    __shared__ int32_t s_ids[kTileEntries];
    __shared__ int32_t s_st;
    const int tile = blockIdx.x, tid = threadIdx.x;
    const int tok0 = tile * sh.tile_tokens;
    const int n = min(sh.tile_tokens, sh.n_tok - tok0) * sh.K;
    const int32_t *src = ids + (int64_t)tok0 * sh.K;
    for (int e = tid; e < sh.E; e += kPlanThreads) s_hist[e] = 0;
    for (int i = tid; i < n; i += kPlanThreads) s_ids[i] = src[i];
    if (tid == 0) s_st = 0;
    __syncthreads();
    int st = 0;
    for (int i = tid; i < n; i += kPlanThreads) {
        const int e = s_ids[i];
        if (e < 0 || e >= sh.E) {
            st |= MOONEP_STATUS_BAD_ID;
            continue;
        }
        const int k = i % sh.K, base = i - k;
        for (int k2 = 0; k2 < k; ++k2)
            if (s_ids[base + k2] == e) st |= MOONEP_STATUS_REPEAT_ID;
        atomicAdd(&s_hist[e], 1);
    }
    if (st) atomicOr(&s_st, st);
    __syncthreads();
    int32_t *out = tile_counts + (int64_t)tile * sh.E;
    for (int e = tid; e < sh.E; e += kPlanThreads) out[e] = s_hist[e];
    if (tid == 0) tile_status[tile] = s_st;
}

// ---------------------------------------------------------------- k_scan
// Lane = expert of a 64-expert column block; the 16 waves split the tiles into
// 16 contiguous runs. Pass 1 sums each run, the runs are prefixed in LDS, pass 2
// rewrites each count as the exclusive prefix over earlier tiles.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void k_scan(PlanShape sh,
                                                       int32_t *__restrict__ tile_counts,
                                                       int32_t *__restrict__ T) {
    __shared__ int32_t s_part[kScanThreads / 64][64];
    const int lane = lane_id(), w = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + lane;
    const int nw = kScanThreads / 64;
    const int run = (sh.n_tiles + nw - 1) / nw;
    const int t0 = min(w * run, sh.n_tiles), t1 = min(t0 + run, sh.n_tiles);
    int sum = 0;
    if (e < sh.E) {
#pragma unroll 8
        for (int t = t0; t < t1; ++t) sum += tile_counts[(int64_t)t * sh.E + e];
    }
    s_part[w][lane] = sum;
    __syncthreads();
    int prefix = 0, total = 0;
    for (int i = 0; i < nw; ++i) {
        const int v = s_part[i][lane];
        prefix += i < w ? v : 0;
        total += v;
    }
    if (e < sh.E) {
        int running = prefix;
#pragma unroll 8
        for (int t = t0; t < t1; ++t) {
            int32_t *c = tile_counts + (int64_t)t * sh.E + e;
            const int v = *c;
            *c = running;
            running += v;
        }
        if (w == 0) T[e] = total;
    }
}

// ---------------------------------------------------------------- k_solve
__global__ __launch_bounds__(kSolveThreads) void k_solve(PlanShape sh, PlanPtrs p) {
    __shared__ int s_cum[kMaxE + 1];    // exclusive prefix of T over all experts
    __shared__ int s_ovpre[kMaxE + 1];  // exclusive prefix of each expert's overflow
    __shared__ int s_nzpre[kMaxE + 1];  // exclusive prefix of (overflow > 0)
    __shared__ int s_ovlist[kMaxE];     // experts with overflow, ascending
    __shared__ int s_listE[kMaxE + kMaxR];
    __shared__ int s_keep[kMaxR], s_Dpre[kMaxR + 1], s_dbeg[kMaxR], s_dend[kMaxR];
    __shared__ int s_nzlo[kMaxR], s_ppre[kMaxR + 1];
    __shared__ int s_w[17];
    __shared__ int s_status;

    const int tid = threadIdx.x;
    const int E = sh.E, R = sh.R, G = sh.G, SK = sh.SK;
    if (tid == 0) s_status = 0;
    __syncthreads();

    // 1. histogram totals, tile status, maxT, maxvio
    const int Te = tid < E ? p.T[tid] : 0;
    int st = 0;
    for (int t = tid; t < sh.n_tiles; t += kSolveThreads) st |= p.tile_status[t];
    if (st) atomicOr(&s_status, st);
    const int maxT = block_max(Te, s_w);

    // 2. home offsets and load. Expert e lives on rank e / G.
    int totT;
    const int cum = block_excl_scan(Te, s_w, totT);
    if (tid < E) s_cum[tid] = cum;
    if (tid == 0) s_cum[E] = totT;
    __syncthreads();
    int hoff = 0;
    if (tid < E) {
        hoff = cum - s_cum[(tid / G) * G];
        p.hoff[tid] = hoff;
    }
    int Lr = 0, keep = 0, O = 0, D = 0;
    if (tid < R) {
        Lr = s_cum[(tid + 1) * G] - s_cum[tid * G];
        keep = min(Lr, SK);
        O = Lr - keep;
        D = SK - keep;
        p.L[tid] = Lr;
        p.keep[tid] = keep;
        p.O[tid] = O;
        p.D[tid] = D;
        s_keep[tid] = keep;
    }

    // 3. water-fill prefix sums
    int totO, totD;
    const int opre = block_excl_scan(O, s_w, totO);
    const int dpre = block_excl_scan(D, s_w, totD);
    if (tid < R) {
        p.Opre[tid] = opre;
        p.Dpre[tid] = dpre;
        s_Dpre[tid] = dpre;
    }
    if (tid == 0) {
        p.Opre[R] = totO;
        p.Dpre[R] = totD;
        s_Dpre[R] = totD;
    }

    // 4. each expert's overflow interval [ovpre, ovpre + ov) in the global
    //    overflow order (home rank, expert, token, k) -- with contiguous homes
    //    that order is simply expert order.
    int ov = 0;
    if (tid < E) ov = max(hoff + Te, SK) - max(hoff, SK);
    int totOV, totNZ;
    const int ovpre = block_excl_scan(ov, s_w, totOV);
    const int nzpre = block_excl_scan(ov > 0 ? 1 : 0, s_w, totNZ);
    if (tid < E) {
        s_ovpre[tid] = ovpre;
        s_nzpre[tid] = nzpre;
        if (ov > 0) s_ovlist[nzpre] = tid;
    }
    if (tid == 0) {
        s_ovpre[E] = totOV;
        s_nzpre[E] = totNZ;
    }
    __syncthreads();

    // 5. pieces per deficit rank: overflowing experts whose interval meets the
    //    rank's filled deficit interval [dbeg, dend).
    int np = 0;
    if (tid < R) {
        const int dbeg = min(s_Dpre[tid], totO), dend = min(s_Dpre[tid + 1], totO);
        s_dbeg[tid] = dbeg;
        s_dend[tid] = dend;
        if (dend > dbeg) {
            const int elo = upper_bound(s_ovpre, E + 1, dbeg) - 1;
            const int ehi = upper_bound(s_ovpre, E + 1, dend - 1) - 1;
            np = s_nzpre[ehi + 1] - s_nzpre[elo];
            s_nzlo[tid] = s_nzpre[elo];
        }
        p.n_dup[tid] = np;
    }
    int P, M;
    const int ppre = block_excl_scan(np, s_w, P);
    const int mpre = block_excl_scan(tid < R ? min(np, sh.B) : 0, s_w, M);
    if (tid < R) {
        s_ppre[tid] = ppre;
        p.mat_pre[tid] = mpre;
        if (np > sh.B) atomicOr(&s_status, MOONEP_STATUS_OVER_B);
    }
    if (tid == 0) {
        s_ppre[R] = P;
        p.mat_pre[R] = M;
        p.n_list[0] = P;
    }
    __syncthreads();

    // 6. one thread per piece: rank-major order equals (expert, rank) order
    //    because both interval families are increasing.
    const int sp = G + sh.dcap + 1, se = G + sh.dcap;
    for (int q = tid; q < P; q += kSolveThreads) {
        const int r = upper_bound(s_ppre, R + 1, q) - 1;
        const int b = q - s_ppre[r];
        const int e = s_ovlist[s_nzlo[r] + b];
        const int js = max(s_ovpre[e], s_dbeg[r]);
        const int je = min(s_ovpre[e + 1], s_dend[r]);
        const int start = s_keep[r] + js - s_Dpre[r];
        const int64_t rb = (int64_t)r * sh.dcap + b;
        p.dup_expert[rb] = e;
        p.dup_start[rb] = start;
        p.dup_count[rb] = je - js;
        p.list_expert[q] = e;
        p.list_rank[q] = r;
        p.list_b[q] = b;
        p.seg_ptr[(int64_t)r * sp + G + b] = start;
        p.seg_expert[(int64_t)r * se + G + b] = e;
        s_listE[q] = e;
    }
    __syncthreads();

    // 7. CSR of the list over experts; experts with duplicates = overflowing experts
    for (int e = tid; e <= E; e += kSolveThreads) p.dup_ptr[e] = lower_bound(s_listE, P, e);
    for (int i = tid; i < totNZ; i += kSolveThreads) p.xlist[i] = s_ovlist[i];

    // 8. home segments and the end of each rank's filled rows
    if (tid < E) {
        const int r = tid / G, i = tid - r * G;
        p.seg_ptr[(int64_t)r * sp + i] = min(hoff, SK);
        p.seg_expert[(int64_t)r * se + i] = tid;
    }
    if (tid < R) p.seg_ptr[(int64_t)tid * sp + G + np] = keep + (s_dend[tid] - s_dbeg[tid]);

    __syncthreads();
    if (tid == 0) {
        p.n_x[0] = totNZ;
        p.maxT[0] = maxT;
        p.maxvio[0] = (double)((int64_t)maxT * E) / (double)sh.n_ent - 1.0;
        p.status[0] = s_status;
    }
}

// ---------------------------------------------------------------- k_assign
__global__ __launch_bounds__(kPlanThreads) void k_assign(const int32_t *__restrict__ ids,
                                                         PlanShape sh, PlanPtrs p) {
    __shared__ int32_t s_ids[kTileEntries];
    __shared__ int32_t s_hist[kWaves][kMaxE];
    __shared__ int32_t s_Dpre[kMaxR + 1], s_Opre[kMaxR + 1], s_keep[kMaxR];
    const int tile = blockIdx.x, tid = threadIdx.x;
    const int lane = lane_id(), w = tid >> 6;
    const int E = sh.E, R = sh.R, SK = sh.SK;
    const int tok0 = tile * sh.tile_tokens;
    const int n = min(sh.tile_tokens, sh.n_tok - tok0) * sh.K;
    const int64_t a0 = (int64_t)tok0 * sh.K;

    for (int i = tid; i < n; i += kPlanThreads) s_ids[i] = ids[a0 + i];
    for (int i = tid; i < kWaves * E; i += kPlanThreads) s_hist[i / E][i % E] = 0;
    for (int r = tid; r <= R; r += kPlanThreads) {
        s_Dpre[r] = p.Dpre[r];
        s_Opre[r] = p.Opre[r];
        if (r < R) s_keep[r] = p.keep[r];
    }
    __syncthreads();

    // each wave owns a contiguous run of whole 64-entry chunks of the tile
    const int per = ((n + kWaves - 1) / kWaves + 63) & ~63;
    const int beg = min(w * per, n), end = min(beg + per, n);

    // pass 1: per-wave expert counts
    for (int i = beg + lane; i < end; i += 64) {
        const int e = s_ids[i];
        if (e >= 0 && e < E) atomicAdd(&s_hist[w][e], 1);
    }
    __syncthreads();
    // per-wave bases: earlier tiles + home offset + earlier waves of this tile
    const int32_t *tbase = p.tile_counts + (int64_t)tile * E;
    for (int e = tid; e < E; e += kPlanThreads) {
        int base = tbase[e] + p.hoff[e];
        for (int v = 0; v < kWaves; ++v) {
            const int c = s_hist[v][e];
            s_hist[v][e] = base;
            base += c;
        }
    }
    __syncthreads();

    // pass 2: chunks of 64 entries in order; rank among equal ids of the chunk
    for (int c0 = beg; c0 < end; c0 += 64) {
        const int i = c0 + lane;
        const int e = i < end ? s_ids[i] : -1;
        const bool valid = e >= 0 && e < E;
        uint64_t mask = __ballot(valid);
        for (int bit = 0; bit < sh.id_bits; ++bit) {
            const bool set = valid && ((e >> bit) & 1);
            const uint64_t bb = __ballot(set);
            mask &= set ? bb : ~bb;
        }
        if (valid) {
            const int below = __builtin_amdgcn_mbcnt_hi(
                (uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
            const int base = s_hist[w][e];
            const int h = base + below;
            if (lane == 63 - __clzll((long long)mask)) s_hist[w][e] = base + __popcll(mask);
            const int r = e / sh.G;
            int slot;
            if (h < SK) {
                slot = r * SK + h;
            } else {
                const int j = s_Opre[r] + (h - SK);
                const int r2 = min(upper_bound(s_Dpre, R + 1, j) - 1, R - 1);
                slot = r2 * SK + s_keep[r2] + (j - s_Dpre[r2]);
            }
            // A correct plan always lands inside the buffer; the guard only keeps a
            // broken invariant from turning into a wild store.
            if ((unsigned)slot < (unsigned)sh.n_ent) {
                p.dst[a0 + i] = slot;
                p.src[slot] = (int32_t)(a0 + i);
            } else {
                p.dst[a0 + i] = -1;
            }
        } else if (i < end) {
            p.dst[a0 + i] = -1;
        }
    }

    // Tails of the plan tables and unfilled slots, spread over the whole grid.
    const int64_t gt = (int64_t)blockIdx.x * kPlanThreads + tid;
    const int64_t gn = (int64_t)gridDim.x * kPlanThreads;
    const int sp = sh.G + sh.dcap + 1, se = sh.G + sh.dcap;
    const int64_t ntab = (int64_t)R * sh.dcap;
    for (int64_t x = gt; x < ntab; x += gn) {
        const int r = (int)(x / sh.dcap), j = (int)(x - (int64_t)r * sh.dcap);
        if (j >= p.n_dup[r]) {
            p.dup_expert[x] = -1;
            p.dup_start[x] = -1;
            p.dup_count[x] = 0;
            p.seg_ptr[(int64_t)r * sp + sh.G + 1 + j] = -1;
            p.seg_expert[(int64_t)r * se + sh.G + j] = -1;
        }
    }
    const int P = p.n_list[0];
    for (int64_t x = P + gt; x < sh.pcap; x += gn) {
        p.list_expert[x] = -1;
        p.list_rank[x] = -1;
        p.list_b[x] = -1;
    }
    // slots that receive nothing (only when some ids were dropped)
    const int totO = s_Opre[R], totD = s_Dpre[R];
    for (int64_t j = totO + gt; j < totD; j += gn) {
        const int r2 = upper_bound(s_Dpre, R + 1, (int)j) - 1;
        p.src[(int64_t)r2 * SK + s_keep[r2] + (j - s_Dpre[r2])] = -1;
    }
}

}  // namespace

hipError_t launch_plan(const PlanShape &sh, const int32_t *ids, const PlanPtrs &p,
                       hipStream_t st) {
    hipLaunchKernelGGL(k_count, dim3(sh.n_tiles), dim3(kPlanThreads), 0, st, ids, sh,
                       p.tile_counts, p.tile_status);
    hipLaunchKernelGGL(k_scan, dim3((sh.E + 63) / 64), dim3(kScanThreads), 0, st, sh,
                       p.tile_counts, p.T);
    hipLaunchKernelGGL(k_solve, dim3(1), dim3(kSolveThreads), 0, st, sh, p);
    hipLaunchKernelGGL(k_assign, dim3(sh.n_tiles), dim3(kPlanThreads), 0, st, ids, sh, p);
    return hipGetLastError();
}

}  // namespace moonep
