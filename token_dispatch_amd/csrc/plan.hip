// Plan kernels for gfx950: the online redundant-expert plan of one step.
//
// The method (news.hamidun.com EN, "How MoonEP works"): every rank receives
// exactly S*K (token, k) assignments whatever the routing skew, by scheduling a
// few duplicate experts from the current router output. Skew is measured as
// maxvio = max_e(T_e / Tbar) - 1 ("Why expert parallelism is needed", same page;
// blog.schoergendorfer.com, "The problem MoonEP targets").
//
// Every grid is fixed by the dims alone (no host round trip). The plan runs as
// four launches, k_count, k_scan, k_solve (or k_solve_bounded), k_assign, or as
// two: k_count, then k_plan_fused, in which every workgroup gathers all tiles'
// counts, runs the whole solve itself and assigns its own tile (no hand-over
// between workgroups); the layout takes two where the counts are few enough.
//   k_count   one workgroup per token tile: one thread per token holds the
//             token's ids in registers, checks them and counts them into the
//             tile's expert histogram in LDS, written to tile_counts[tile][E].
//   k_scan    one workgroup per 64 experts: exclusive scan of tile_counts down
//             the tiles (in place) and the column totals T[e].
//   k_solve   one workgroup (the water-fill): home offsets, home load, keep /
//             overflow / deficit and their prefix sums, then the duplicates as
//             the intersections of each expert's overflow interval with each
//             rank's deficit interval (a merge of two sorted boundary lists),
//             and all plan tables.
//   k_solve_bounded  one workgroup (at most B duplicates per rank where it can):
//             the same head, then each overloaded rank's overflow from its
//             largest experts and one wave placing the pieces rank by rank.
//   k_assign  one 1024-thread workgroup per token tile, for either plan: the
//             stable position of every entry inside its expert (tile base +
//             per-wave base + in-wave rank from per-token LDS atomics, or
//             bit-sliced ballots for small K and repeated ids), then its
//             slot -- a home slot below kept[e], else an offset into the one
//             piece of its expert that holds its overflow row -- and the
//             inverse map, walking the tile's entries in expert order so that
//             the inverse-map stores come in runs of consecutive slots.
//
// Why this is exact: entry a's position inside expert e is the number of
// earlier entries with id e. That count is split as (earlier tiles) + (earlier
// waves of this tile) + (earlier entries of this wave), each an integer count
// taken in entry order.
#include <atomic>
#include <cstddef>

#include "internal.h"

namespace moonep {
namespace {

constexpr int kAssignThreads = 1024;
constexpr int kAssignWaves = kAssignThreads / 64;
constexpr int kChunks = kTileEntries / kAssignThreads;  // 64-entry chunks per assign wave
constexpr int kMaxIdBits = 10;                          // bits of an expert id below kMaxE
static_assert(kTileEntries % kAssignThreads == 0, "a tile is a whole number of chunks per wave");
static_assert(kMaxE <= kAssignThreads && kMaxR <= kAssignThreads && kMaxE <= kSolveThreads &&
                  kMaxR <= kSolveThreads,
              "one expert or rank per thread (the E-th / R-th prefix entries come from thread 0)");
static_assert((1 << kMaxIdBits) >= kMaxE, "ids fit the ballot bit slices");
static_assert(kSolveThreads == kAssignThreads, "assign uses the solve's block scan");
static_assert(kTileEntries <= (1 << 22), "an in-tile index and an id share a word");
static_assert(kTileEntries < (1 << 16), "a tile's count of one expert fits 16 bits");
static_assert(kMaxE <= 1024 && (kMaxE & (kMaxE - 1)) == 0, "expert ids fit the 10-bit field of a packed placement key");

// The plan kernels take a few hundred bytes of arguments (the plan's table
// pointers). The compiler cannot hold them all in scalar registers, so it reads
// them from the argument segment in several rounds, each waiting for its
// scalar-cache misses before the next. Reading one word of every 64-byte line
// of the arguments first, and waiting for them together, takes all those misses
// in one round trip; the later reads hit the scalar cache.
struct SolveArgs {
    PlanShape sh;
    PlanPtrs p;
};
struct TileArgs {
    const int32_t *ids;
    PlanShape sh;
    PlanPtrs p;
};

template <class Args>
__device__ __forceinline__ void touch_kernargs() {
    constexpr int kLines = (int)((sizeof(Args) + 63) / 64);
    const uint32_t *ka = (const uint32_t *)__builtin_amdgcn_kernarg_segment_ptr();
    uint32_t x = 0;
#pragma unroll
    for (int l = 0; l < kLines; ++l) x ^= ka[l * 16];
    asm volatile("" ::"s"(x));
}

// The kernel's PlanPtrs argument, read through a pointer into the argument
// segment that the compiler cannot see through. Read as the parameter itself,
// every pointer is loaded once at the start and held in scalar registers for the
// whole kernel, which does not fit (the bounded fused kernel spilled 83 of them
// to vector lanes); read this way, each is loaded from the scalar cache where it
// is used.
typedef __attribute__((address_space(4))) const PlanPtrs ConstPlanPtrs;
template <class Args>
__device__ __forceinline__ const PlanPtrs &plan_ptrs() {
    ConstPlanPtrs *pp = (ConstPlanPtrs *)((const __attribute__((address_space(4))) char *)
                                              __builtin_amdgcn_kernarg_segment_ptr() +
                                          offsetof(Args, p));
    asm volatile("" : "+s"(pp));
    return *(const PlanPtrs *)pp;
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Inclusive scan over the 64 lanes of a wave with DPP moves (no LDS): shifts by
// 1, 2, 4, 8 inside each 16-lane row, then lane 15 of a row into the next row
// and lane 31 into the upper two rows. Lanes with no source get 0 added.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// Maximum over the 64 lanes, in every lane: DPP shifts inside each 16-lane row,
// then rows 0 -> 1 and 1 -> 2,3 broadcasts (lane 63 ends with the maximum).
__device__ __forceinline__ int wave_reduce_max(int x) {
    constexpr int kLo = -2147483647 - 1;
    x = max(x, __builtin_amdgcn_update_dpp(kLo, x, 0x111, 0xf, 0xf, false));  // row_shr:1
    x = max(x, __builtin_amdgcn_update_dpp(kLo, x, 0x112, 0xf, 0xf, false));  // row_shr:2
    x = max(x, __builtin_amdgcn_update_dpp(kLo, x, 0x114, 0xf, 0xf, false));  // row_shr:4
    x = max(x, __builtin_amdgcn_update_dpp(kLo, x, 0x118, 0xf, 0xf, false));  // row_shr:8
    x = max(x, __builtin_amdgcn_update_dpp(kLo, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
    x = max(x, __builtin_amdgcn_update_dpp(kLo, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return __builtin_amdgcn_readlane(x, 63);
}

// Exclusive scans of NV values per thread over the 1024-thread workgroup, all
// in one pass (two barriers): each wave scans itself, publishes its total, then
// scans the 16 totals itself. s_w needs 16 * NV ints. Every thread must call it;
// tot[i] receives the total of value i. LDS written before the call is visible
// to every thread after it.
template <int NV>
__device__ void block_excl_scan(const int *v, int *res, int *tot, int *s_w) {
    constexpr int NW = kSolveThreads / 64;
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    int inc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) inc[i] = wave_incl_scan(v[i]);
    if (lane == 63) {
#pragma unroll
        for (int i = 0; i < NV; ++i) s_w[i * NW + w] = inc[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int ti = wave_incl_scan(lane < NW ? s_w[i * NW + lane] : 0);
        const int before = w == 0 ? 0 : __builtin_amdgcn_readlane(ti, w - 1);
        res[i] = inc[i] - v[i] + before;
        tot[i] = __builtin_amdgcn_readlane(ti, NW - 1);
    }
    __syncthreads();  // s_w is free for the next scan
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

// Sum of v over each aligned group of GS consecutive lanes (GS = 1, 2, 4, 8 or
// 16), in every lane of the group, by DPP moves inside rows; every lane of the
// group must be active.
template <int GS>
__device__ __forceinline__ int group_sum(int v) {
    if constexpr (GS >= 2) v += __builtin_amdgcn_mov_dpp(v, 0xb1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
    if constexpr (GS >= 4) v += __builtin_amdgcn_mov_dpp(v, 0x4e, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
    if constexpr (GS >= 8) v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xf, 0xf, false);  // row_half_mirror
    if constexpr (GS >= 16) v += __builtin_amdgcn_mov_dpp(v, 0x140, 0xf, 0xf, false); // row_mirror
    return v;
}

// Lanes per item when the workgroup counts, for each of n items, the keys that
// order before it: 16 for 16 < n <= 64 items (four keys per lane), else one
// thread per item.
__device__ __forceinline__ int count_group(int n) { return n > 16 && n <= kSolveThreads / 16 ? 16 : 1; }

// The keys among k[0 .. n) that order before x (before(k[j], x)), counted by
// the gs lanes of the item (count_group); every lane of the group gets the total.
template <class Key, class Before>
__device__ __forceinline__ int group_count(const Key *k, int n, Key x, int gs, Before before) {
    int c = 0;
    if (gs == 16) {
        const int sub = (int)threadIdx.x & 15;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = sub + 16 * u;
            const bool b = before(k[min(j, n - 1)], x);
            c += j < n && b ? 1 : 0;
        }
        return group_sum<16>(c);
    }
#pragma unroll 8
    for (int j = 0; j < n; ++j) c += before(k[j], x) ? 1 : 0;
    return c;
}

// ---------------------------------------------------------------- k_count
// KMAX: a power of two >= K; TPT tokens per thread cover the largest tile any K
// in (KMAX/2, KMAX] gives. All of a thread's ids are loaded before any is used.
// Repeated ids: each thread keeps a set of 1024 bits in LDS for its current
// token (rows of 36 words: 16-byte aligned, and lanes 1 row apart start 4 banks
// apart). Bit e is set with an atomic OR that returns the word's old value, so
// a token's K ids cost K atomics instead of K(K-1)/2 compares; the atomics of
// one lane run in program order, so a second e sees the first one's bit.
constexpr int kSeenWords = kMaxE / 32;
constexpr int kSeenStride = kSeenWords + 4;
static_assert(kMaxE % 128 == 0, "a seen-set row is whole 16-byte groups");
constexpr int tpt_of(int kmax) {
    return (kTileEntries / (kmax == 1 ? 1 : kmax / 2 + 1) + kPlanThreads - 1) / kPlanThreads;
}

// U16: the counts are stored as 16-bit words (a tile holds at most kTileEntries
// <= 65535 entries), for the two-launch plan whose every workgroup reads them all;
// the four-launch plan keeps 32-bit words, which k_scan turns into prefixes.
template <int KMAX, bool U16>
__global__ __launch_bounds__(kPlanThreads) void k_count(const int32_t *__restrict__ ids,
                                                        PlanShape sh,
                                                        int32_t *__restrict__ tile_counts,
                                                        int32_t *__restrict__ tile_status) {
    constexpr int TPT = tpt_of(KMAX);
    __shared__ int32_t s_hist[kMaxE];
    __shared__ int32_t s_st;
    __shared__ __align__(16) uint32_t s_seen[kPlanThreads * kSeenStride];
    const int tile = blockIdx.x, tid = threadIdx.x;
    const int K = sh.K;
    const int tok0 = tile * sh.tile_tokens;
    const int ntok = min(sh.tile_tokens, sh.n_tok - tok0);
    for (int e = tid; e < sh.E; e += kPlanThreads) s_hist[e] = 0;
    if (tid == 0) s_st = 0;
    uint32_t *seen = s_seen + tid * kSeenStride;  // this thread's own row: no barrier needed
    if (KMAX > 1) {
#pragma unroll
        for (int q = 0; q < kSeenWords; q += 4)
            *reinterpret_cast<uint4 *>(seen + q) = make_uint4(0u, 0u, 0u, 0u);
    }

    // 16-byte loads when a token's ids are whole 16-byte groups (ids is 16-byte aligned)
    const bool vec = KMAX >= 4 && (K & 3) == 0;
    int v[TPT][KMAX];
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
        const int t = tid + j * kPlanThreads;
        const int32_t *src = ids + (int64_t)(tok0 + t) * K;
#pragma unroll
        for (int k = 0; k < KMAX; k += 4) {
            if (vec) {
                int4 q = make_int4(-1, -1, -1, -1);
                if (t < ntok && k < K) q = *reinterpret_cast<const int4 *>(src + k);
                v[j][k] = q.x;
                if (k + 1 < KMAX) v[j][k + 1] = q.y;
                if (k + 2 < KMAX) v[j][k + 2] = q.z;
                if (k + 3 < KMAX) v[j][k + 3] = q.w;
            } else {
#pragma unroll
                for (int u = 0; u < 4 && k + u < KMAX; ++u)
                    v[j][k + u] = (t < ntok && k + u < K) ? src[k + u] : -1;
            }
        }
    }
    __syncthreads();

    int st = 0;
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
        if (j * kPlanThreads + (tid & ~63) >= ntok) break;  // no token left in this wave
        const bool tok_ok = tid + j * kPlanThreads < ntok;
        // no branches between the atomics, so they all issue before the first
        // returned value is waited for; an absent or bad id adds 0 to word 0
        uint32_t got[KMAX], bitv[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int e = v[j][k];
            const bool in = tok_ok && k < K;
            const bool ok = in && e >= 0 && e < sh.E;
            if (in && !ok) st |= MOONEP_STATUS_BAD_ID;
            const int ee = ok ? e : 0;
            bitv[k] = ok ? 1u << (e & 31) : 0u;
            if (KMAX > 1) got[k] = atomicOr(&seen[ee >> 5], bitv[k]);
            atomicAdd(&s_hist[ee], ok ? 1 : 0);
        }
        if (KMAX > 1) {
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if (got[k] & bitv[k]) st |= MOONEP_STATUS_REPEAT_ID;
            // clear the words this token touched, ready for the thread's next token
            if (j + 1 < TPT) {
#pragma unroll
                for (int k = 0; k < KMAX; ++k)
                    if (bitv[k]) seen[v[j][k] >> 5] = 0u;
            }
        }
    }
    if (st) atomicOr(&s_st, st);
    __syncthreads();
    if constexpr (U16) {
        uint16_t *out = reinterpret_cast<uint16_t *>(tile_counts) + (int64_t)tile * sh.E;
        for (int e = tid; e < sh.E; e += kPlanThreads) out[e] = (uint16_t)s_hist[e];
    } else {
        int32_t *out = tile_counts + (int64_t)tile * sh.E;
        for (int e = tid; e < sh.E; e += kPlanThreads) out[e] = s_hist[e];
    }
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
    constexpr int kCache = 32;  // a wave's run of tiles kept in registers between the passes
    __shared__ int32_t s_part[kScanThreads / 64][64];
    const int lane = lane_id(), w = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + lane;
    const int nw = kScanThreads / 64;
    const int run = (sh.n_tiles + nw - 1) / nw;
    const int t0 = min(w * run, sh.n_tiles), t1 = min(t0 + run, sh.n_tiles);
    const bool cached = t1 - t0 <= kCache;  // the same for every lane of the wave
    int v[kCache];
    int sum = 0;
    if (cached) {
        // all of the run's loads in flight at once
#pragma unroll
        for (int u = 0; u < kCache; ++u)
            v[u] = (e < sh.E && t0 + u < t1) ? tile_counts[(int64_t)(t0 + u) * sh.E + e] : 0;
#pragma unroll
        for (int u = 0; u < kCache; ++u) sum += v[u];
    } else if (e < sh.E) {
#pragma unroll 8
        for (int t = t0; t < t1; ++t) sum += tile_counts[(int64_t)t * sh.E + e];
    }
    s_part[w][lane] = sum;
    __syncthreads();
    int prefix = 0, total = 0;
    for (int i = 0; i < nw; ++i) {
        const int x = s_part[i][lane];
        prefix += i < w ? x : 0;
        total += x;
    }
    if (e < sh.E) {
        int running = prefix;
        if (cached) {
#pragma unroll
            for (int u = 0; u < kCache; ++u) {
                if (t0 + u < t1) tile_counts[(int64_t)(t0 + u) * sh.E + e] = running;
                running += v[u];
            }
        } else {
#pragma unroll 8
            for (int t = t0; t < t1; ++t) {
                int32_t *c = tile_counts + (int64_t)t * sh.E + e;
                const int x = *c;
                *c = running;
                running += x;
            }
        }
        if (w == 0) T[e] = total;
    }
}

// ---------------------------------------------------------------- solve
// The part both solves share: tile status bits and maxT (into *s_status,
// *s_maxT), T in LDS, the exclusive prefix of T (s_cum), home offsets and home
// load, keep / overflow / deficit per rank (written to the plan and to s_keep,
// s_O, s_D). Every thread of the 1024-thread workgroup must call it, with Te =
// T of expert threadIdx.x (0 beyond E) and st = its share of the OR of the
// tiles' status words.
struct Head {
    int Te, hoff, keep, O, D;
};

__device__ Head solve_head(const PlanShape &sh, const PlanPtrs &p, int Te, int st, int *s_T,
                           int *s_cum, int *s_keep, int *s_O, int *s_D, int *s_w, int *s_status,
                           int *s_maxT) {
    const int tid = threadIdx.x, lane = lane_id();
    const int E = sh.E, R = sh.R, G = sh.G, SK = sh.SK;
    Head h{};
    h.Te = Te;
    if (tid == 0) {
        *s_status = 0;
        *s_maxT = 0;
    }
    if (tid < E) s_T[tid] = h.Te;
    __syncthreads();
    if (st) atomicOr(s_status, st);
    {
        const int m = wave_reduce_max(h.Te);
        if (lane == 0) atomicMax(s_maxT, m);
    }
    // home offsets and load; expert e lives on rank e / G
    int cum, totT;
    block_excl_scan<1>(&h.Te, &cum, &totT, s_w);
    if (tid < E) s_cum[tid] = cum;
    if (tid == 0) s_cum[E] = totT;
    __syncthreads();
    if (tid < E) {
        h.hoff = cum - s_cum[(tid / G) * G];
        p.hoff[tid] = h.hoff;
    }
    if (tid < R) {
        const int Lr = s_cum[(tid + 1) * G] - s_cum[tid * G];
        h.keep = min(Lr, SK);
        h.O = Lr - h.keep;
        h.D = SK - h.keep;
        p.L[tid] = Lr;
        p.keep[tid] = h.keep;
        p.O[tid] = h.O;
        p.D[tid] = h.D;
        s_keep[tid] = h.keep;
        s_O[tid] = h.O;
        s_D[tid] = h.D;
    }
    __syncthreads();
    return h;
}

// The plan's scalar results, written once every atomic on them has landed.
__device__ void solve_tail(const PlanShape &sh, const PlanPtrs &p, int n_x, const int *s_status,
                           const int *s_maxT) {
    if (threadIdx.x == 0) {
        const int maxT = *s_maxT;
        p.n_x[0] = n_x;
        p.maxT[0] = maxT;
        p.maxvio[0] = (double)((int64_t)maxT * sh.E) / (double)sh.n_ent - 1.0;
        p.status[0] = *s_status;
    }
}

// ---------------------------------------------------------------- LDS of the solves
// Both solves carve their LDS from one int block sized to the problem (E, R,
// pcap); the same function gives the host the size and the device the arrays.
struct LdsCarve {
    int32_t *base;
    int off;
    __host__ __device__ int32_t *take(int n) {
        int32_t *r = base ? base + off : nullptr;
        off += n;
        return r;
    }
};

constexpr int kScanScratch = (kSolveThreads / 64 + 1) * 4;  // block_excl_scan<NV <= 4>

struct WfLds {
    int32_t *T, *cum, *ovpre, *ovp, *ovlist, *listE;
    int32_t *keep, *O, *D, *Dpre, *dbeg, *dend, *nzlo, *rnp, *ppre, *w, *scal;
};

__host__ __device__ inline int wf_lds(int E, int R, int pcap, int32_t *base, WfLds *o) {
    LdsCarve c{base, 0};
    WfLds l;
    l.T = c.take(E);
    l.cum = c.take(E + 1);     // exclusive prefix of T over all experts
    l.ovpre = c.take(E + 1);   // exclusive prefix of each expert's overflow
    l.ovp = c.take(E + 1);     // overflow starts of the experts with overflow, then the total
    l.ovlist = c.take(E);      // experts with overflow, ascending
    l.listE = c.take(pcap);
    l.keep = c.take(R);
    l.O = c.take(R);
    l.D = c.take(R);
    l.Dpre = c.take(R + 1);
    l.dbeg = c.take(R);
    l.dend = c.take(R);
    l.nzlo = c.take(R);
    l.rnp = c.take(R);         // pieces per rank
    l.ppre = c.take(R + 1);
    l.w = c.take(kScanScratch);
    l.scal = c.take(4);        // status, maxT
    if (o) *o = l;
    return c.off;
}

struct BdLds {
    uint64_t *bkey, *ekey;
    int32_t *T, *cum, *kc, *ov, *xl, *bin, *binD, *binK, *keep, *O, *D, *nd, *first, *fill;
    int32_t *pe, *pr, *pstart, *pcnt, *pjj, *pkey, *skey, *w, *scal;
};

__host__ __device__ inline int bd_lds(int E, int R, int pcap, int32_t *base, BdLds *o) {
    LdsCarve c{base, 0};
    BdLds l;
    l.bkey = reinterpret_cast<uint64_t *>(c.take(2 * R));  // first: 8-byte aligned
    l.ekey = reinterpret_cast<uint64_t *>(c.take(2 * E));  // expert order within a rank
    l.T = c.take(E);
    l.cum = c.take(E + 1);
    l.kc = c.take(E + 1);      // exclusive prefix of kept rows
    l.ov = c.take(E);          // overflow rows of each expert
    l.xl = c.take(E);          // overflowing experts in id order
    l.bin = c.take(R + 1);     // deficit ranks in fill order: rank, D, keep
    l.binD = c.take(R + 1);
    l.binK = c.take(R + 1);
    l.keep = c.take(R);
    l.O = c.take(R);
    l.D = c.take(R);
    l.nd = c.take(R);
    l.first = c.take(R);
    l.fill = c.take(R);
    l.pe = c.take(pcap);
    l.pr = c.take(pcap);
    l.pstart = c.take(pcap);
    l.pcnt = c.take(pcap);
    l.pjj = c.take(pcap);
    l.pkey = c.take(pcap);
    l.skey = c.take(pcap);
    l.w = c.take(kScanScratch);
    l.scal = c.take(4);        // status, maxT, pieces, error
    if (o) *o = l;
    return c.off;
}

inline size_t solve_lds_bytes(const PlanShape &sh, bool bounded) {
    const int n = bounded ? bd_lds(sh.E, sh.R, sh.pcap, nullptr, nullptr)
                          : wf_lds(sh.E, sh.R, sh.pcap, nullptr, nullptr);
    return sizeof(int32_t) * (size_t)n;
}

// ---------------------------------------------------------------- water-fill solve
// One 1024-thread workgroup; smem holds wf_lds() ints. Returns the plan's status word.
__device__ __forceinline__ int solve_waterfill(const PlanShape &sh, const PlanPtrs &p,
                                                int32_t *smem, int Te, int st) {
    WfLds L;
    wf_lds(sh.E, sh.R, sh.pcap, smem, &L);
    int *const s_T = L.T, *const s_cum = L.cum, *const s_ovpre = L.ovpre, *const s_ovp = L.ovp;
    int *const s_ovlist = L.ovlist, *const s_listE = L.listE, *const s_keep = L.keep, *const s_O = L.O;
    int *const s_D = L.D, *const s_Dpre = L.Dpre, *const s_dbeg = L.dbeg, *const s_dend = L.dend;
    int *const s_nzlo = L.nzlo, *const s_rnp = L.rnp, *const s_ppre = L.ppre, *const s_w = L.w;
    int &s_status = L.scal[0], &s_maxT = L.scal[1];

    const int tid = threadIdx.x;
    const int E = sh.E, R = sh.R, G = sh.G, SK = sh.SK;
    const Head h = solve_head(sh, p, Te, st, s_T, s_cum, s_keep, s_O, s_D, s_w, &s_status, &s_maxT);
    // each expert's overflow: the part of its home list [hoff, hoff + T) at or
    // beyond S*K; in the global overflow order (home rank, expert, token, k) --
    // with contiguous homes simply expert order -- it is [ovpre, ovpre + ov).
    // Its first kept = T - ov entries stay home, from row min(hoff, S*K).
    const int ov = tid < E ? max(h.hoff + h.Te, SK) - max(h.hoff, SK) : 0;
    if (tid < E) {
        p.kept[tid] = h.Te - ov;
        p.koff[tid] = min(h.hoff, SK);
    }

    // the water-fill prefix sums of O and D, and of ov and (ov > 0), in one pass
    int v4[4] = {h.O, h.D, ov, ov > 0 ? 1 : 0}, pre[4], tot[4];
    block_excl_scan<4>(v4, pre, tot, s_w);
    const int totO = tot[0], totD = tot[1], totNZ = tot[3];
    if (tid < R) {
        p.Opre[tid] = pre[0];
        p.Dpre[tid] = pre[1];
        s_Dpre[tid] = pre[1];
    }
    if (tid < E) {
        s_ovpre[tid] = pre[2];
        if (ov > 0) {
            s_ovlist[pre[3]] = tid;
            s_ovp[pre[3]] = pre[2];
        }
    }
    if (tid == 0) {
        p.Opre[R] = totO;
        p.Dpre[R] = totD;
        s_Dpre[R] = totD;
        s_ovpre[E] = tot[2];
        s_ovp[totNZ] = tot[2];
    }
    __syncthreads();

    // pieces per deficit rank: the overflowing experts whose interval meets the
    // rank's filled deficit interval [dbeg, dend), found in the compact list of
    // overflow starts. Threads 2r and 2r + 1 search for the two ends at once;
    // every lane runs the same iterations, so the pair exchange sees both.
    for (int x0 = 0; x0 < 2 * R; x0 += kSolveThreads) {
        const int x = x0 + tid, r = x >> 1;
        int dbeg = 0, dend = 0, k = 0;
        if (r < R) {
            dbeg = min(s_Dpre[r], totO);
            dend = min(s_Dpre[r + 1], totO);
            if (dend > dbeg) k = upper_bound(s_ovp, totNZ + 1, (x & 1) ? dend - 1 : dbeg) - 1;
        }
        const int k_end = __builtin_amdgcn_mov_dpp(k, 0xb1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]: lane ^ 1
        if (r < R && (x & 1) == 0) {
            s_dbeg[r] = dbeg;
            s_dend[r] = dend;
            s_nzlo[r] = k;
            s_rnp[r] = dend > dbeg ? k_end - k + 1 : 0;
        }
    }
    __syncthreads();
    int np = 0;
    if (tid < R) {
        np = s_rnp[tid];
        p.n_dup[tid] = np;
        if (np > sh.B) atomicOr(&s_status, MOONEP_STATUS_OVER_B);
    }
    // pieces, materialised duplicates and empty slots (only with dropped ids) per rank
    int v3[3] = {np, tid < R ? min(np, sh.B) : 0, tid < R ? h.D - (s_dend[tid] - s_dbeg[tid]) : 0};
    int ppre[3], ptot[3];
    block_excl_scan<3>(v3, ppre, ptot, s_w);
    const int P = ptot[0];
    if (tid < R) {
        s_ppre[tid] = ppre[0];
        p.mat_pre[tid] = ppre[1];
        p.upre[tid] = ppre[2];
    }
    if (tid == 0) {
        s_ppre[R] = P;
        p.mat_pre[R] = ptot[1];
        p.upre[R] = ptot[2];
        p.n_list[0] = P;
    }
    __syncthreads();

    // one thread per piece: rank-major order equals (expert, rank) order
    // because both interval families are increasing
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
        p.piece_js[q] = js - s_ovpre[e];  // first overflow index of the piece within its expert
        p.pslot[q] = r * SK + start;
        p.pcnt[q] = je - js;
        p.seg_ptr[(int64_t)r * sp + G + b] = start;
        p.seg_expert[(int64_t)r * se + G + b] = e;
        s_listE[q] = e;
    }
    __syncthreads();

    // CSR of the list over experts; experts with duplicates = overflowing experts
    for (int e = tid; e <= E; e += kSolveThreads) p.dup_ptr[e] = lower_bound(s_listE, P, e);
    for (int i = tid; i < totNZ; i += kSolveThreads) p.xlist[i] = s_ovlist[i];

    // home segments and the end of each rank's filled rows
    if (tid < E) {
        const int r = tid / G, i = tid - r * G;
        p.seg_ptr[(int64_t)r * sp + i] = min(h.hoff, SK);
        p.seg_expert[(int64_t)r * se + i] = tid;
    }
    if (tid < R) p.seg_ptr[(int64_t)tid * sp + G + np] = h.keep + (s_dend[tid] - s_dbeg[tid]);
    solve_tail(sh, p, totNZ, &s_status, &s_maxT);
    return s_status;
}

// T (from k_scan) and this thread's share of the tiles' status words.
__device__ __forceinline__ void solve_inputs(const PlanShape &sh, const PlanPtrs &p, int &Te, int &st) {
    const int tid = threadIdx.x;
    Te = tid < sh.E ? p.T[tid] : 0;
    st = 0;
    for (int t = tid; t < sh.n_tiles; t += kSolveThreads) st |= p.tile_status[t];
}

__global__ __launch_bounds__(kSolveThreads) void k_solve(PlanShape sh, PlanPtrs) {
    extern __shared__ int32_t smem[];
    touch_kernargs<SolveArgs>();
    const PlanPtrs &p = plan_ptrs<SolveArgs>();
    int Te, st;
    solve_inputs(sh, p, Te, st);
    solve_waterfill(sh, p, smem, Te, st);
}

// ---------------------------------------------------------------- k_solve_bounded
// The plan that keeps at most B duplicates per rank where it can: an overloaded
// rank overflows its largest experts first (T descending, then id); deficit ranks
// are filled one at a time, largest deficit first (then rank id); a rank's
// pieces 1 .. B-1 are the largest remaining overflow that fits whole (then lowest
// id), or if none fits a piece of the largest one; its B-th piece is a piece of
// the smallest remaining overflow that fills the room (then lowest id), or if none
// is that large the largest one whole, after which the rank goes on the same way
// over its budget (MOONEP_STATUS_OVER_B). Exact S*K rows per rank and the minimum
// number of moved rows hold as for the water-fill.
//
// Every rule picks a number of rows first and then the lowest id among the
// overflows with that many rows left, so one placement step is a few wave-wide
// maximum reductions over the overflows, which wave 0 holds in registers
// (kMaxE / 64 per lane): two when (rows, id) packs into one 31-bit key, three
// otherwise. Up to 64 overflows with packed keys take place_pieces_sorted, where
// a step is a few ballots over the overflows kept in order.
constexpr int kItemsPerLane = kMaxE / 64;

struct PlaceArgs {
    int n_items, n_bins, B, cap;
    const int *s_xl, *s_ov;
    const int *s_bin, *s_binD, *s_binK;  // deficit ranks in fill order: rank, D, keep
    int *s_first, *s_nd, *s_fill, *s_pe, *s_pr, *s_pstart, *s_pcnt, *s_pjj;
    int *s_rkey, *s_rbin;  // place_pieces_sorted's records: key taken, place of the rank
    const int *s_okey;     // place_pieces_sorted's overflow keys, already in order
};

// The placement, run by one wave: ranks in fill order, pieces by the rules
// above. Lane l holds overflows l, l + 64, ... of the id-ordered list in NS
// register slots (so within a lane a lower slot is a lower id); the lane that
// holds the chosen overflow records the piece. Returns the number of pieces, or
// -(pieces + 1) if the piece tables ran out of room (cannot happen: pieces <=
// overflowing experts + deficit ranks - 1).
template <int NS, bool PACKED>
__device__ __forceinline__ int place_pieces(const PlaceArgs &a) {
    constexpr int kLo = -2147483647 - 1;
    constexpr int kVmax = (1 << 21) - 1;  // PACKED: rows left fit 21 bits, ids 10
    const int lane = lane_id();
    int lv[NS], lid[NS], lov[NS];  // rows left (0: placed), expert id (-1: none), overflow rows
#pragma unroll
    for (int c = 0; c < NS; ++c) {
        const int i = c * 64 + lane;
        lid[c] = i < a.n_items ? a.s_xl[i] : -1;
        lov[c] = lid[c] >= 0 ? a.s_ov[lid[c]] : 0;
        lv[c] = lov[c];
    }
    int n = a.n_items, np = 0;
    int r_nx = a.s_bin[0], D_nx = a.s_binD[0], K_nx = a.s_binK[0];  // the next rank, loaded ahead
    for (int bi = 0; bi < a.n_bins && n > 0; ++bi) {
        const int r = r_nx, D = D_nx, keep = K_nx;
        if (bi + 1 < a.n_bins) {
            r_nx = a.s_bin[bi + 1];
            D_nx = a.s_binD[bi + 1];
            K_nx = a.s_binK[bi + 1];
        }
        int room = D, used = 0;
        if (lane == 0) a.s_first[r] = np;
        while (room > 0 && n > 0) {
            if (np >= a.cap) return -(np + 1);
            const bool fit_rule = used < a.B - 1;
            int v, e;
            if constexpr (PACKED) {
                // one key per overflow, larger = preferred: (rows, lowest id) for the
                // whole-fit rule and the largest, (fewest rows, lowest id) for the
                // filling rule; -1 = not a candidate
                int pk = -1, fk = -1;
#pragma unroll
                for (int c = 0; c < NS; ++c) {
                    const int x = lv[c], low = (kMaxE - 1) - lid[c];
                    const int big = (x << 10) | low;
                    fk = max(fk, x > 0 ? big : -1);
                    if (fit_rule) pk = max(pk, x > 0 && x <= room ? big : -1);
                    else pk = max(pk, x >= room ? ((kVmax - x) << 10) | low : -1);
                }
                const int pm = wave_reduce_max(pk), fm = wave_reduce_max(fk);
                const int k = pm >= 0 ? pm : fm;
                e = (kMaxE - 1) - (k & (kMaxE - 1));
                v = pm >= 0 && !fit_rule ? kVmax - (k >> 10) : k >> 10;
            } else {
                // this lane's candidate numbers of rows: by the rule (as a maximum)
                // and the largest; then the lowest id with that many rows left
                int pv = kLo, fv = kLo;
#pragma unroll
                for (int c = 0; c < NS; ++c) {
                    fv = max(fv, lv[c]);
                    if (fit_rule) pv = max(pv, lv[c] > 0 && lv[c] <= room ? lv[c] : kLo);
                    else pv = max(pv, lv[c] >= room ? -lv[c] : kLo);
                }
                const int pm = wave_reduce_max(pv), fm = wave_reduce_max(fv);
                v = pm != kLo ? (fit_rule ? pm : -pm) : fm;
                int key = -1;
#pragma unroll
                for (int c = NS - 1; c >= 0; --c) key = lv[c] == v ? 0x7fffffff - lid[c] : key;
                e = 0x7fffffff - wave_reduce_max(key);
            }
            const int t = min(v, room);
            int jj0 = -1;
#pragma unroll
            for (int c = 0; c < NS; ++c) {
                const bool mine = lid[c] == e;
                jj0 = mine ? lov[c] - v : jj0;
                lv[c] = mine ? v - t : lv[c];
            }
            if (jj0 >= 0) {
                a.s_pe[np] = e;
                a.s_pr[np] = r;
                a.s_pstart[np] = keep + (D - room);
                a.s_pcnt[np] = t;
                a.s_pjj[np] = jj0;
            }
            ++np;
            room -= t;
            ++used;
            n -= v == t ? 1 : 0;
        }
        if (lane == 0) {
            a.s_nd[r] = used;
            a.s_fill[r] = D - room;
        }
    }
    return np;
}

template <int NS>
__device__ __forceinline__ int place_pieces(const PlaceArgs &a, bool packed) {
    return packed ? place_pieces<NS, true>(a) : place_pieces<NS, false>(a);
}

// v_writelane_b32: reg with lane `lane` set to val (both wave-uniform).
__device__ int amdgcn_writelane(int val, int lane, int reg) __asm("llvm.amdgcn.writelane.i32");

// The same placement for at most 64 overflows whose rows fit 21 bits, deficits
// of at most 2^21 rows and B <= 63, with the overflows kept sorted across the
// wave instead of searched: lane p holds the overflow at position p of the order
// (rows left descending, then id ascending) as the key
// ((rows - 1) << 10) | (kMaxE - 1 - id), read from s_okey in that order, and a
// wave-uniform mask has a bit per lane whose overflow still has rows. The rank's free room is kept as
// T = room * 1024 - 1, so that "rows <= room" is "key <= T" and a full rank
// (T = -1) matches no key. Every rule then reads the first (or last) set bit
// of a ballot:
//   largest that fits whole  first live lane with key <= T
//   largest                  first live lane
//   smallest that fills      the last live lane with key > T - 1024 has the
//                            fewest rows; the first live lane with those rows
//                            has the lowest id among them
// A piece that cuts an overflow (always a rank's last) moves its key down past
// the live keys that are now larger, the keys between moving up one lane (a
// whole-wave DPP shift). A step is a short chain of scalar work around one
// ballot and one lane read, and it records only the key it took and the rank's
// place in fill order (lane = piece mod 64, written to LDS in windows of up to
// 64); every other table follows from those two afterwards, in parallel
// (expand_sorted_pieces), because all but a rank's last piece are whole.
struct PieceRegs {
    int key, bin;
};

// records of pieces from .. to - 1 (at most 64), piece q in lane q mod 64
__device__ __forceinline__ void flush_window(const PlaceArgs &a, const PieceRegs &g, int from, int to) {
    const int q = from + ((lane_id() - from) & 63);
    if (q < to) {
        a.s_rkey[q] = g.key;
        a.s_rbin[q] = g.bin;
    }
}

// Exit codes of run_ranks.
constexpr int kRunDone = 0, kRunStop = 1, kRunFlush = 2, kRunFill = 3;

// The common steps of place_pieces_sorted in one block of scalar and vector
// instructions, with no memory access: ranks from bi on, each taking whole fits
// (its pieces 1 .. B-1) and, when none fits, a piece of the largest overflow,
// which ends the rank. Written out by hand because the compiler's rendering of
// the branches adds a scalar copy or select to every step, and a step is a
// chain of dependent scalar and lane operations. On entry B >= 2, bi < bstop,
// live != 0 and np <= npmax; D of rank bi is in lane bi mod 64 of Dl, and
// bstop is the next multiple of 64 after bi or the number of ranks, if less.
// Stops with
//   kRunDone    no overflow is left
//   kRunStop    bi reached bstop (Dl holds the wrong ranks, or every rank is done)
//   kRunFlush   the next rank could overrun the 64 piece records (np > npmax)
//   kRunFill    rank bi has taken B-1 whole fits and has room T left
// The only backward branches follow an increment of used (< B-1) or of
// bi (< bstop), so the block always ends. Lane selects come from scalar
// instructions only (M0 for lane writes, whose data is the one SGPR operand a
// vector instruction may read); an SGPR read by a lane write is written by a
// lane read at least two instructions earlier, and a DPP read of key follows
// s_nop 1.
__device__ __forceinline__ void run_ranks(int &key, PieceRegs &g, int Dl, int lane, uint64_t &live,
                                          int &bi, int &np, int bstop, int fitp, int npmax, int &T,
                                          int &code) {
    uint64_t m, t;
    int L, k, A, D, used;
    int vn;
    // every scalar operand as a wave-uniform value, as the SGPR constraints need
    auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
    uint64_t lv = ((uint64_t)(uint32_t)uni((int)(live >> 32)) << 32) | (uint32_t)uni((int)live);
    int b = uni(bi), n = uni(np);
    const int nbu = uni(bstop), fitu = uni(fitp), npmu = uni(npmax);
    asm volatile(
        ".Lrank%=:\n"
        "  s_and_b32 %[L], %[bi], 63\n"
        "  v_readlane_b32 %[D], %[dl], %[L]\n"
        "  s_mov_b32 %[used], 0\n"
        "  s_lshl_b32 %[T], %[D], 10\n"
        "  s_add_i32 %[T], %[T], -1\n"
        ".Lfit%=:\n"
        "  v_cmp_ge_i32 vcc, %[T], %[key]\n"
        "  s_and_b64 %[m], vcc, %[live]\n"
        "  s_cbranch_scc0 .Lnofit%=\n"
        "  s_ff1_i32_b64 %[L], %[m]\n"
        "  v_readlane_b32 %[k], %[key], %[L]\n"
        "  s_mov_b32 m0, %[np]\n"
        "  v_writelane_b32 %[gb], %[bi], m0\n"
        "  s_bitset0_b64 %[live], %[L]\n"
        "  v_writelane_b32 %[gk], %[k], m0\n"
        "  s_andn2_b32 %[k], 0xfffffc00, %[k]\n"
        "  s_add_i32 %[np], %[np], 1\n"
        "  s_add_i32 %[T], %[T], %[k]\n"
        "  s_add_i32 %[used], %[used], 1\n"
        "  s_cmp_lt_i32 %[used], %[fitp]\n"
        "  s_cbranch_scc1 .Lfit%=\n"
        "  s_cmp_lt_i32 %[T], 0\n"
        "  s_cbranch_scc1 .Lnext%=\n"
        "  s_cmp_eq_u64 %[live], 0\n"
        "  s_cbranch_scc1 .Ldone%=\n"
        "  s_mov_b32 %[code], 3\n"
        "  s_branch .Lexit%=\n"
        ".Lnofit%=:\n"
        "  s_cmp_lt_i32 %[T], 0\n"
        "  s_cbranch_scc1 .Lnext%=\n"
        "  s_cmp_eq_u64 %[live], 0\n"
        "  s_cbranch_scc1 .Ldone%=\n"
        "  s_ff1_i32_b64 %[L], %[live]\n"
        "  v_readlane_b32 %[k], %[key], %[L]\n"
        "  s_mov_b32 m0, %[np]\n"
        "  v_writelane_b32 %[gb], %[bi], m0\n"
        "  s_add_i32 %[A], %[T], 1\n"
        "  v_writelane_b32 %[gk], %[k], m0\n"
        "  s_add_i32 %[np], %[np], 1\n"
        "  s_sub_i32 %[k], %[k], %[A]\n"
        "  v_cmp_lt_i32 vcc, %[k], %[key]\n"
        "  s_and_b64 %[m], vcc, %[live]\n"
        "  s_bitset0_b64 %[m], %[L]\n"
        "  s_flbit_i32_b64 %[A], %[m]\n"
        "  s_xor_b32 %[A], %[A], 63\n"
        "  s_cmp_le_i32 %[A], %[L]\n"
        "  s_cbranch_scc1 .Linplace%=\n"
        "  s_nop 1\n"
        "  v_mov_b32_dpp %[vn], %[key] wave_shl:1 row_mask:0xf bank_mask:0xf\n"
        "  v_cmp_le_i32 %[t], %[L], %[vl]\n"
        "  v_cmp_gt_i32 vcc, %[A], %[vl]\n"
        "  s_and_b64 vcc, vcc, %[t]\n"
        "  s_sub_i32 %[D], 63, %[A]\n"
        "  s_mov_b32 m0, %[A]\n"
        "  v_cndmask_b32 %[key], %[key], %[vn], vcc\n"
        "  v_writelane_b32 %[key], %[k], m0\n"
        "  s_lshr_b64 %[t], -1, %[D]\n"
        "  s_lshl_b64 %[m], -1, %[L]\n"
        "  s_and_b64 %[t], %[t], %[m]\n"
        "  s_lshr_b64 %[m], %[live], 1\n"
        "  s_and_b64 %[m], %[m], %[t]\n"
        "  s_andn2_b64 %[live], %[live], %[t]\n"
        "  s_or_b64 %[live], %[live], %[m]\n"
        "  s_bitset1_b64 %[live], %[A]\n"
        "  s_branch .Lnext%=\n"
        ".Linplace%=:\n"
        "  s_mov_b32 m0, %[L]\n"
        "  v_writelane_b32 %[key], %[k], m0\n"
        ".Lnext%=:\n"
        "  s_add_i32 %[bi], %[bi], 1\n"
        "  s_cmp_eq_u32 %[bi], %[bstop]\n"
        "  s_cbranch_scc1 .Lstop%=\n"
        "  s_cmp_gt_i32 %[np], %[npmax]\n"
        "  s_cbranch_scc0 .Lrank%=\n"
        "  s_mov_b32 %[code], 2\n"
        "  s_branch .Lexit%=\n"
        ".Lstop%=:\n"
        "  s_mov_b32 %[code], 1\n"
        "  s_branch .Lexit%=\n"
        ".Ldone%=:\n"
        "  s_mov_b32 %[code], 0\n"
        ".Lexit%=:\n"
        : [key] "+v"(key), [gk] "+v"(g.key), [gb] "+v"(g.bin), [live] "+s"(lv), [bi] "+s"(b),
          [np] "+s"(n), [T] "=&s"(T), [code] "=&s"(code), [m] "=&s"(m), [t] "=&s"(t),
          [L] "=&s"(L), [k] "=&s"(k), [A] "=&s"(A), [D] "=&s"(D), [used] "=&s"(used),
          [vn] "=&v"(vn)
        : [dl] "v"(Dl), [vl] "v"(lane), [bstop] "s"(nbu), [fitp] "s"(fitu), [npmax] "s"(npmu)
        : "vcc", "scc", "m0");
    // the results are wave-uniform; say so, or they would be kept per lane
    live = ((uint64_t)(uint32_t)uni((int)(lv >> 32)) << 32) | (uint32_t)uni((int)lv);
    bi = uni(b);
    np = uni(n);
    T = uni(T);
    code = uni(code);
}

__device__ __forceinline__ int place_pieces_sorted(const PlaceArgs &a) {
    const int lane = lane_id();
    const int n0 = __builtin_amdgcn_readfirstlane(a.n_items);
    const int nb = __builtin_amdgcn_readfirstlane(a.n_bins);
    const int fit_pieces = __builtin_amdgcn_readfirstlane(a.B - 1);
    // records a rank adds before its fill steps: its whole fits and one more
    const int need = max(fit_pieces, 0) + 1;
    int key = lane < n0 ? a.s_okey[lane] : 0;
    uint64_t live = n0 >= 64 ? ~0ull : (1ull << n0) - 1;
    constexpr uint64_t kTop = 1ull << 63;

    // No check against the piece tables' room: every piece but a rank's last
    // places an overflow whole, so pieces <= overflows + ranks - 1 < pcap.
    PieceRegs g{0, 0};
    int np = 0, fl = 0;  // pieces placed; pieces whose records are in LDS
    int bi = 0;          // place of the rank in fill order
    auto record = [&](int k) {
        const int slot = np & 63;
        g.key = amdgcn_writelane(k, slot, g.key);
        g.bin = amdgcn_writelane(bi, slot, g.bin);
        ++np;
    };
    // lane j: deficit of the rank at place (bi & ~63) + j
    int Dl = lane < nb ? a.s_binD[lane] : 0;
    while (bi < nb && live != 0) {
        // room for a rank's fit pieces and the step after them
        if (np - fl > 64 - need) {
            flush_window(a, g, fl, np);
            fl = np;
        }
        // Ranks from bi on, while every step is a whole fit or a rank's last
        // piece of the largest overflow; see run_ranks. With B <= 1 a rank has
        // no fit pieces, and every rank takes the fill steps below.
        int T, code = kRunFill;
        if (fit_pieces > 0) {
            const int bstop = min(nb, (bi & ~63) + 64);
            run_ranks(key, g, Dl, lane, live, bi, np, bstop, fit_pieces, fl + 64 - need, T, code);
        } else {
            T = (int)(((unsigned)__builtin_amdgcn_readlane(Dl, bi & 63) << 10) - 1u);
        }
        if (code == kRunDone) break;
        if (code == kRunStop) {
            if (bi < nb) {
                const int j = bi + lane;
                Dl = j < nb ? a.s_binD[j] : 0;
            }
            continue;
        }
        if (code == kRunFlush) continue;
        // kRunFill: rank bi has placed its fit pieces and has room left; the
        // smallest overflow that fills the room (lowest id among those rows), or
        // if none is that large the largest whole
        int L, k;
        bool cut;
        for (;;) {
            if (np - fl == 64) {
                flush_window(a, g, fl, np);
                fl = np;
            }
            const uint64_t ge = __builtin_amdgcn_ballot_w64(key > T - kMaxE) & live;
            const int h = 63 - __builtin_clzll(ge | 1);
            const int kh = __builtin_amdgcn_readlane(key, h) & ~(kMaxE - 1);
            const uint64_t eq =
                __builtin_amdgcn_ballot_w64((unsigned)(key - kh) < (unsigned)kMaxE) & live;
            L = __builtin_ctzll((ge != 0 ? eq : live) | kTop);
            k = __builtin_amdgcn_readlane(key, L);
            record(k);
            cut = k > T;  // more rows than room: the piece fills the rank
            if (cut) break;
            T -= (k | (kMaxE - 1)) + 1;
            live &= ~(1ull << L);
            if (T < 0 || live == 0) break;
        }
        if (cut) {
            // the overflow keeps rows: its key drops below the live keys of the
            // lanes up to A, which move up one lane with their bits
            const int k2 = k - (T + 1);
            const uint64_t gt = __builtin_amdgcn_ballot_w64(key > k2) & live & ~(1ull << L);
            const int A = gt != 0 ? 63 - __builtin_clzll(gt) : -1;
            if (A > L) {
                // DPP wave_shl:1: lane i reads lane i + 1
                const int next = __builtin_amdgcn_update_dpp(key, key, 0x130, 0xf, 0xf, false);
                key = lane >= L && lane < A ? next : key;
                key = amdgcn_writelane(k2, A, key);
                const uint64_t span = (~0ull >> (63 - A)) & (~0ull << L);  // bits L..A
                live = (live & ~span) | ((live >> 1) & span) | (1ull << A);
            } else {
                key = amdgcn_writelane(k2, L, key);
            }
        }
        ++bi;
        if ((bi & 63) == 0 && bi < nb) {
            const int j = bi + lane;
            Dl = j < nb ? a.s_binD[j] : 0;
        }
    }
    flush_window(a, g, fl, np);
    return np;
}

// The tables of the pieces place_pieces_sorted recorded (key taken, place of the
// rank in fill order), one thread per piece: a rank's pieces are consecutive,
// all but its last take their overflow whole, and the last takes what is left
// of the rank's deficit if that is less.
__device__ __forceinline__ void expand_sorted_pieces(const PlaceArgs &a, int P) {
    for (int q = threadIdx.x; q < P; q += kSolveThreads) {
        const int k = a.s_rkey[q], bi = a.s_rbin[q];
        int j = q, before = 0;  // the rank's first piece; rows of its pieces before q
        while (j > 0 && a.s_rbin[j - 1] == bi) {
            --j;
            before += (a.s_rkey[j] >> 10) + 1;
        }
        const int v = (k >> 10) + 1, e = (kMaxE - 1) - (k & (kMaxE - 1));
        const int r = a.s_bin[bi], cnt = min(v, a.s_binD[bi] - before);
        a.s_pe[q] = e;
        a.s_pr[q] = r;
        a.s_pstart[q] = a.s_binK[bi] + before;
        a.s_pcnt[q] = cnt;
        a.s_pjj[q] = a.s_ov[e] - v;  // first overflow row of the piece
        if (j == q) a.s_first[r] = q;
        if (q + 1 == P || a.s_rbin[q + 1] != bi) {
            a.s_nd[r] = q - j + 1;
            a.s_fill[r] = before + cnt;
        }
    }
}

// One 1024-thread workgroup; smem holds bd_lds() ints. Returns the plan's status word.
__device__ __forceinline__ int solve_bounded(const PlanShape &sh, const PlanPtrs &p,
                                              int32_t *smem, int Te, int st) {
    BdLds L;
    bd_lds(sh.E, sh.R, sh.pcap, smem, &L);
    uint64_t *const s_bkey = L.bkey;
    int *const s_T = L.T, *const s_cum = L.cum, *const s_kc = L.kc, *const s_ov = L.ov, *const s_xl = L.xl;
    int *const s_bin = L.bin, *const s_binD = L.binD, *const s_binK = L.binK, *const s_keep = L.keep;
    int *const s_O = L.O, *const s_D = L.D, *const s_nd = L.nd, *const s_first = L.first;
    int *const s_fill = L.fill, *const s_pe = L.pe, *const s_pr = L.pr, *const s_pstart = L.pstart;
    int *const s_pcnt = L.pcnt, *const s_pjj = L.pjj, *const s_pkey = L.pkey, *const s_skey = L.skey;
    int *const s_w = L.w;
    int &s_status = L.scal[0], &s_maxT = L.scal[1], &s_np = L.scal[2], &s_err = L.scal[3];

    const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    const int E = sh.E, R = sh.R, G = sh.G, B = sh.B;
    // each expert's place in its rank's overflow order (T descending, then id)
    // as one key, T in the high word; solve_head's first barrier publishes them
    uint64_t *const s_ekey = L.ekey;
    if (tid < E) s_ekey[tid] = ((uint64_t)(uint32_t)Te << 32) | (uint32_t)~tid;
    const Head h = solve_head(sh, p, Te, st, s_T, s_cum, s_keep, s_O, s_D, s_w, &s_status, &s_maxT);

    // 1. overflow of each overloaded rank, from its largest experts
    int ov = 0;
    if (tid < E) {
        const int r = tid / G;
        const uint64_t mine = s_ekey[tid];
        int before = 0;  // rows of the rank's experts that come before this one
        // branch-free and unrolled, so that the LDS reads go out together
#pragma unroll 8
        for (int e2 = r * G; e2 < (r + 1) * G; ++e2) {
            const uint64_t k2 = s_ekey[e2];
            before += k2 > mine ? (int)(k2 >> 32) : 0;
        }
        ov = min(max(s_O[r] - before, 0), h.Te);
        s_ov[tid] = ov;
    }
    if (tid < R)  // deficit descending, then rank ascending
        s_bkey[tid] = h.D > 0 ? ((uint64_t)(uint32_t)h.D << 32) | (uint32_t)(0x7fffffff - tid) : 0;
    const int kept = tid < E ? h.Te - ov : 0;
    int kv[3] = {kept, ov > 0 ? 1 : 0, tid < R && h.D > 0 ? 1 : 0}, kpre[3], ktot[3];
    block_excl_scan<3>(kv, kpre, ktot, s_w);
    const int n_items = ktot[1], n_bins = ktot[2];
    // up to 64 overflows with rows below 2^21, deficits of at most 2^21 rows and
    // B <= 63 take place_pieces_sorted
    const bool packed = s_maxT < (1 << 21);  // every overflow's rows fit a 21-bit key field
    const bool sorted = n_items <= 64 && packed && sh.SK <= (1 << 21) && B <= 63;
    int *const s_ukey = s_T, *const s_okey = s_cum;  // T and its prefix are spent
    if (tid < E) {
        s_kc[tid] = kpre[0];
        if (ov > 0) {
            s_xl[kpre[1]] = tid;
            if (sorted) s_ukey[kpre[1]] = ((ov - 1) << 10) | (kMaxE - 1 - tid);
        }
    }
    if (tid == 0) {
        s_kc[E] = ktot[0];
        s_np = 0;
        s_err = 0;
    }
    {  // each rank's place in fill order: the ranks whose key is larger, counted
       // by a group of lanes per rank
        const int gs = count_group(R), r = tid / gs;
        if (r < R) {
            const uint64_t mine = s_bkey[r];
            const int pos = group_count(s_bkey, R, mine, gs,
                                        [](uint64_t a, uint64_t b) { return a > b; });
            if ((tid & (gs - 1)) == 0 && mine != 0) {
                s_bin[pos] = r;
                s_binD[pos] = s_D[r];
                s_binK[pos] = s_keep[r];
            }
        }
    }
    int v2[2] = {h.O, h.D}, dpre[2], dtot[2];
    block_excl_scan<2>(v2, dpre, dtot, s_w);  // also orders the writes above
    if (sorted) {  // the overflow keys in descending order (they are distinct)
        const int gs = count_group(n_items), i = tid / gs;
        if (i < n_items) {
            const int x = s_ukey[i];
            const int pos = group_count(s_ukey, n_items, x, gs, [](int a, int b) { return a > b; });
            if ((tid & (gs - 1)) == 0) s_okey[pos] = x;
        }
    }
    if (tid < R) {
        p.Opre[tid] = dpre[0];
        p.Dpre[tid] = dpre[1];
        s_nd[tid] = 0;
        s_fill[tid] = 0;
        s_first[tid] = 0;
    }
    if (tid == 0) {
        p.Opre[R] = dtot[0];
        p.Dpre[R] = dtot[1];
    }
    if (tid < E) {
        p.kept[tid] = kept;
        p.koff[tid] = kpre[0] - s_kc[(tid / G) * G];
    }
    __syncthreads();

    // 2. placement (wave 0), with as many register slots per lane as the overflows need
    const PlaceArgs a{n_items, n_bins, B, sh.pcap, s_xl, s_ov, s_bin, s_binD, s_binK, s_first, s_nd,
                      s_fill, s_pe, s_pr, s_pstart, s_pcnt, s_pjj, s_pkey, s_skey, s_okey};
    const int nslots = (n_items + 63) >> 6;
    if (w == 0) {
        int np;
        if (sorted) np = place_pieces_sorted(a);
        else if (nslots <= 1) np = place_pieces<1, false>(a);
        else if (nslots <= 2) np = place_pieces<2>(a, packed);
        else if (nslots <= 4) np = place_pieces<4>(a, packed);
        else if (nslots <= 8) np = place_pieces<8>(a, packed);
        else np = place_pieces<kItemsPerLane>(a, packed);
        if (lane == 0) {
            s_np = np < 0 ? -np - 1 : np;
            s_err = np < 0 ? 1 : 0;
        }
    }
    __syncthreads();

    // 3. tables: per rank (pieces in placement order), the list by (expert, rank)
    const int P = s_np;
    if (sorted) {
        expand_sorted_pieces(a, P);
        __syncthreads();
    }
    const int sp = G + sh.dcap + 1, se = G + sh.dcap;
    for (int q = tid; q < P; q += kSolveThreads) {
        const int r = s_pr[q], e = s_pe[q], b = q - s_first[r];
        s_pkey[q] = e * R + r;  // one piece per (expert, rank)
        if (b >= sh.dcap) continue;  // cannot happen: a rank takes each expert at most once
        const int64_t rb = (int64_t)r * sh.dcap + b;
        p.dup_expert[rb] = e;
        p.dup_start[rb] = s_pstart[q];
        p.dup_count[rb] = s_pcnt[q];
        p.seg_ptr[(int64_t)r * sp + G + b] = s_pstart[q];
        p.seg_expert[(int64_t)r * se + G + b] = e;
    }
    int nd = 0;
    if (tid < R) {
        nd = s_nd[tid];
        p.n_dup[tid] = nd;
        if (nd > B) atomicOr(&s_status, MOONEP_STATUS_OVER_B);
        if (s_err) atomicOr(&s_status, MOONEP_STATUS_BAD_ID);
    }
    int mv[2] = {tid < R ? min(nd, B) : 0, tid < R ? h.D - s_fill[tid] : 0}, mpre[2], mtot[2];
    block_excl_scan<2>(mv, mpre, mtot, s_w);  // also orders the key writes above
    if (tid < R) {
        p.mat_pre[tid] = mpre[0];
        p.upre[tid] = mpre[1];
    }
    if (tid == 0) {
        p.mat_pre[R] = mtot[0];
        p.upre[R] = mtot[1];
        p.n_list[0] = P;
    }
    {  // the list: each piece's place among the (expert, rank) keys, counted by a
       // group of lanes per piece
        const int gs = count_group(P);
        for (int q = tid / gs; q < P; q += kSolveThreads / gs) {
            const int key = s_pkey[q];
            const int pos = group_count(s_pkey, P, key, gs, [](int a, int b) { return a < b; });
            if ((tid & (gs - 1)) == 0) {
                s_skey[pos] = key;
                p.list_expert[pos] = s_pe[q];
                p.list_rank[pos] = s_pr[q];
                p.list_b[pos] = q - s_first[s_pr[q]];
                p.piece_js[pos] = s_pjj[q];
                p.pslot[pos] = s_pr[q] * sh.SK + s_pstart[q];
                p.pcnt[pos] = s_pcnt[q];
            }
        }
    }
    __syncthreads();
    // CSR over experts: pieces of expert e are the keys in [e*R, (e+1)*R)
    for (int e = tid; e <= E; e += kSolveThreads) p.dup_ptr[e] = lower_bound(s_skey, P, e * R);
    for (int i = tid; i < n_items; i += kSolveThreads) p.xlist[i] = s_xl[i];
    if (tid < E) {
        const int r = tid / G, i = tid - r * G;
        p.seg_ptr[(int64_t)r * sp + i] = kpre[0] - s_kc[r * G];
        p.seg_expert[(int64_t)r * se + i] = tid;
    }
    if (tid < R && nd <= sh.dcap) p.seg_ptr[(int64_t)tid * sp + G + nd] = h.keep + s_fill[tid];
    solve_tail(sh, p, n_items, &s_status, &s_maxT);
    return s_status;
}

__global__ __launch_bounds__(kSolveThreads) void k_solve_bounded(PlanShape sh, PlanPtrs) {
    extern __shared__ int32_t smem[];
    touch_kernargs<SolveArgs>();
    const PlanPtrs &p = plan_ptrs<SolveArgs>();
    int Te, st;
    solve_inputs(sh, p, Te, st);
    solve_bounded(sh, p, smem, Te, st);
}

// ---------------------------------------------------------------- assign
// A tile has tile_chunks (1 to kChunks) 64-entry chunks per wave: wave w takes
// entries [w*n, w*n + n), n = tile_chunks*64, lane l holding entry w*n + c*64 + l
// of chunk c. Both plans place entries the
// same way: an entry's position among its expert's entries (token, then k order)
// below kept[e] is a home row from koff[e] on; position kept[e] + jj is overflow
// row jj of the expert, in the one piece whose range [jj0, jj0 + count) holds it.
//
// LDS (ints): s_pos, the per-wave counts and then running positions of every
// expert (kAssignWaves / 2 * E; waves 2m and 2m+1 share a word, low and high 16
// bits -- a tile has at most 4096 entries, so a half never carries into the
// other), then the plan tables the placement reads.
struct AsgTables {
    int32_t *tbase;    // entries of e in earlier tiles
    int32_t *kept;     // entries of e kept at home
    int32_t *kslot;    // first home slot of e
    int32_t *dup_ptr;  // pieces of e: [dup_ptr[e], dup_ptr[e+1])
    int32_t *pjj;      // first overflow row of each piece within its expert
    int32_t *pcnt;     // rows of each piece
    int32_t *pslot;    // first slot of each piece
    int32_t *upre;     // R + 1: exclusive prefix of empty slots per rank
    int32_t *toff;     // first index of e in this tile's expert-ordered list
    uint32_t *ord;     // the tile's valid entries in (expert, token, k) order: i << 10 | e
    int32_t *scan_w;   // block scan scratch
};

__host__ __device__ inline int asg_tables(int E, int R, int pcap, int cap, int32_t *base,
                                          AsgTables *o) {
    LdsCarve c{base, 0};
    AsgTables t;
    t.tbase = c.take(E);
    t.kept = c.take(E);
    t.kslot = c.take(E);
    t.dup_ptr = c.take(E + 1);
    t.pjj = c.take(pcap);
    t.pcnt = c.take(pcap);
    t.pslot = c.take(pcap);
    t.upre = c.take(R + 1);
    t.toff = c.take(E);
    t.ord = reinterpret_cast<uint32_t *>(c.take(cap));
    t.scan_w = c.take(kAssignWaves + 1);
    if (o) *o = t;
    return c.off;
}

// Entries a tile's lanes can hold (a tile has at most that many).
__host__ __device__ inline int tile_cap(const PlanShape &sh) { return sh.tile_chunks * kAssignThreads; }

// s_pos also holds the tile's slots by entry once the positions are spent.
__host__ __device__ inline int pos_ints(const PlanShape &sh) {
    const int counts = (kAssignWaves / 2) * sh.E;
    return counts > tile_cap(sh) ? counts : tile_cap(sh);
}

inline size_t assign_lds_bytes(const PlanShape &sh) {
    return sizeof(int32_t) *
           (size_t)(pos_ints(sh) + asg_tables(sh.E, sh.R, sh.pcap, tile_cap(sh), nullptr, nullptr));
}

struct Tile {
    int tile;   // index of the tile
    int n;      // entries in it
    int64_t a0; // its first entry
};

__device__ __forceinline__ Tile tile_of(const PlanShape &sh, int tile) {
    const int tok0 = tile * sh.tile_tokens;
    return Tile{tile, min(sh.tile_tokens, sh.n_tok - tok0) * sh.K, (int64_t)tok0 * sh.K};
}

__device__ __forceinline__ void load_ids(const PlanShape &sh, const int32_t *__restrict__ ids,
                                         const Tile &t, int (&idv)[kChunks]) {
    const int w = threadIdx.x >> 6, lane = lane_id();
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        const int i = w * (sh.tile_chunks * 64) + c * 64 + lane;
        idv[c] = c < sh.tile_chunks && i < t.n ? ids[t.a0 + i] : -1;
    }
}

// The plan tables the placement needs, fetched into registers with every load
// in flight at once, and written to LDS later (no barrier), so that their
// latency passes while the ranks are taken. tile_counts[tile] already holds the
// exclusive prefix over earlier tiles. The whole piece table is fetched, with
// no dependent loads: only entries below the list length are ever looked up
// (through dup_ptr).
static_assert(kMaxE + kMaxR <= 2 * kAssignThreads, "two piece-table entries per thread");
struct TableRegs {
    int tbase, kept, koff, dup_ptr, upre;  // expert (rank) threadIdx.x
    int dup_end, upre_end;                 // dup_ptr[E] and upre[R]
    int pjj[2], pcnt[2], pslot[2];         // list entries threadIdx.x and + kAssignThreads
};

// Every thread issues every load (indices clamped into range), so that the
// number of loads in flight is the same on every path and the ranks can start
// as soon as the ids are in, with the table loads still outstanding.
__device__ __forceinline__ TableRegs fetch_tables(const PlanShape &sh, const PlanPtrs &p, int tile,
                                                  bool scanned_base) {
    const int tid = threadIdx.x, E = sh.E, R = sh.R;
    const int e = min(tid, E - 1), r = min(tid, R);
    TableRegs g;
    g.tbase = scanned_base ? p.tile_counts[(int64_t)tile * E + e] : 0;
    g.kept = p.kept[e];
    g.koff = p.koff[e];
    g.dup_ptr = p.dup_ptr[e];
    g.upre = p.upre[r];
    g.dup_end = p.dup_ptr[E];
    g.upre_end = p.upre[R];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int q = min(tid + k * kAssignThreads, sh.pcap - 1);
        g.pjj[k] = p.piece_js[q];
        g.pcnt[k] = p.pcnt[q];
        g.pslot[k] = p.pslot[q];
    }
    return g;
}

__device__ __forceinline__ void store_tables(const PlanShape &sh, const TableRegs &g,
                                             const AsgTables &t) {
    const int tid = threadIdx.x, E = sh.E, R = sh.R;
    if (tid < E) {
        t.tbase[tid] = g.tbase;
        t.kept[tid] = g.kept;
        t.kslot[tid] = (tid / sh.G) * sh.SK + g.koff;
        t.dup_ptr[tid] = g.dup_ptr;
    }
    if (tid < R) t.upre[tid] = g.upre;
    if (tid == 0) {
        t.dup_ptr[E] = g.dup_end;
        t.upre[R] = g.upre_end;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int q = tid + k * kAssignThreads;
        if (q < sh.pcap) {
            t.pjj[q] = g.pjj[k];
            t.pcnt[q] = g.pcnt[k];
            t.pslot[q] = g.pslot[k];
        }
    }
}

__device__ __forceinline__ void zero_pos(const PlanShape &sh, uint32_t *s_pos) {
#pragma unroll
    for (int m = 0; m < kAssignWaves / 2; ++m)
        if ((int)threadIdx.x < sh.E) s_pos[m * sh.E + threadIdx.x] = 0u;
}

// Pass 1: the stable rank of every entry among its wave's entries of its expert
// ((token, k) order), while the wave's per-expert totals build up in s_pos.
//
// By tokens (K >= 4 and no repeated ids): the K ids of one token are distinct,
// so the lanes of one token can add to their counters in one LDS atomic without
// two of them meeting on a counter, and the value each gets back is the number
// of earlier entries of its expert in the wave. The wave issues its tokens in
// order and LDS runs a wave's operations in issue order. The token of in-tile
// entry i is floor((i + 0.5) / K), taken in binary32: for i < 4096 and K <= 64
// the quotient lies at least 1/128 from an integer and the rounding error is
// below 1e-3, so the floor is exact.
//
// By id bit slices (small K, where a chunk holds many tokens, or repeated ids,
// where two lanes of one atomic could meet): one ballot per id bit finds the
// lanes holding the same id; the lowest of them adds their number and hands
// the count before them back to the others.
__device__ __forceinline__ void rank_entries(const PlanShape &sh, const int (&idv)[kChunks],
                                             bool by_tokens, int (&rank)[kChunks],
                                             uint32_t *s_pos) {
    const int w = threadIdx.x >> 6, lane = lane_id();
    const int half = (w & 1) * 16;
    uint32_t *ctr = s_pos + (w >> 1) * sh.E;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        if (c >= sh.tile_chunks) break;
        const int e = idv[c];
        const bool valid = e >= 0 && e < sh.E;
        uint32_t got = 0;
        if (by_tokens) {
            const int i = w * (sh.tile_chunks * 64) + c * 64 + lane;
            const int tok = (int)(((float)i + 0.5f) * sh.inv_k);
            const int tok0 = __builtin_amdgcn_readlane(tok, 0);
            const int n_sub = __builtin_amdgcn_readlane(tok, 63) - tok0 + 1;
            for (int j = 0; j < n_sub; ++j)
                if (valid && tok - tok0 == j) got = atomicAdd(&ctr[e], 1u << half);
            rank[c] = (int)((got >> half) & 0xffffu);
        } else {
            uint64_t mask = __ballot(valid);
#pragma unroll
            for (int bit = 0; bit < kMaxIdBits; ++bit) {
                if (bit < sh.id_bits) {
                    const bool set = valid && ((e >> bit) & 1);
                    const uint64_t bb = __ballot(set);
                    mask &= set ? bb : ~bb;
                }
            }
            const int lead = __ffsll((unsigned long long)mask) - 1;
            if (valid && lane == lead) got = atomicAdd(&ctr[e], (uint32_t)__popcll(mask) << half);
            const uint32_t base = (uint32_t)__shfl((int)got, lead < 0 ? 0 : lead);
            const int below = __builtin_amdgcn_mbcnt_hi(
                (uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
            rank[c] = (int)((base >> half) & 0xffffu) + below;
        }
    }
}

// Per-wave counts -> running positions relative to the tile base (earlier waves
// of this tile); returns the tile's count of expert threadIdx.x (0 beyond E).
__device__ __forceinline__ int running_positions(const PlanShape &sh, uint32_t *s_pos) {
    uint32_t run = 0;
    if ((int)threadIdx.x < sh.E) {
#pragma unroll
        for (int m = 0; m < kAssignWaves / 2; ++m) {
            const uint32_t word = s_pos[m * sh.E + threadIdx.x];
            const uint32_t lo = word & 0xffffu, hi = word >> 16;
            s_pos[m * sh.E + threadIdx.x] = run | ((run + lo) << 16);
            run += lo + hi;
        }
    }
    return (int)run;
}

// Pass 2: every valid entry goes into the tile's expert-ordered list, at its
// expert's start in the tile + the expert's entries in earlier waves + its rank
// in its wave.
__device__ __forceinline__ void order_entries(const PlanShape &sh, const int (&idv)[kChunks],
                                              const int (&rank)[kChunks], const uint32_t *s_pos,
                                              const AsgTables &tb) {
    const int w = threadIdx.x >> 6, lane = lane_id();
    const int half = (w & 1) * 16;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        if (c >= sh.tile_chunks) break;
        const int e = idv[c];
        if (e >= 0 && e < sh.E) {
            const int i = w * (sh.tile_chunks * 64) + c * 64 + lane;
            const int rel = (int)((s_pos[(w >> 1) * sh.E + e] >> half) & 0xffffu);
            tb.ord[tb.toff[e] + rel + rank[c]] = ((uint32_t)i << 10) | (uint32_t)e;
        }
    }
}

// Pass 3, over the list: consecutive threads take consecutive entries of one
// expert, whose slots are consecutive too, so the stores into the inverse map
// come in runs instead of one cache line per lane. An entry's position p in its
// expert is a home row below kept[e]; above, overflow row p - kept[e] lies in
// exactly one piece of the expert. The slot of entry i also goes to s_dst[i].
__device__ __forceinline__ void place_sorted(const PlanShape &sh, const PlanPtrs &p, const Tile &t,
                                             int n_valid, const AsgTables &tb, int32_t *s_dst) {
    for (int j = threadIdx.x; j < n_valid; j += kAssignThreads) {
        const uint32_t v = tb.ord[j];
        const int i = (int)(v >> 10), e = (int)(v & 1023u);
        const int pos = tb.tbase[e] + (j - tb.toff[e]);
        const int kept = tb.kept[e];
        int slot = -1;
        if (pos < kept) {
            slot = tb.kslot[e] + pos;
        } else {
            const int jj = pos - kept;
            const int q1 = tb.dup_ptr[e + 1];
            for (int q = tb.dup_ptr[e]; q < q1; ++q) {
                const int d = jj - tb.pjj[q];
                if ((unsigned)d < (unsigned)tb.pcnt[q]) {
                    slot = tb.pslot[q] + d;
                    break;
                }
            }
        }
        // A correct plan always lands inside the buffer; the guard only keeps a
        // broken invariant from turning into a wild store.
        if ((unsigned)slot < (unsigned)sh.n_ent) p.src[slot] = (int32_t)(t.a0 + i);
        else slot = -1;
        s_dst[i] = slot;
    }
}

// Pass 4: dst in entry order, whole 64-entry runs per store; -1 for bad ids.
__device__ __forceinline__ void write_dst(const PlanShape &sh, const PlanPtrs &p, const Tile &t,
                                          const int (&idv)[kChunks], const int32_t *s_dst) {
    const int w = threadIdx.x >> 6, lane = lane_id();
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        if (c >= sh.tile_chunks) break;
        const int i = w * (sh.tile_chunks * 64) + c * 64 + lane;
        const int e = idv[c];
        if (i < t.n) p.dst[t.a0 + i] = (e >= 0 && e < sh.E) ? s_dst[i] : -1;
    }
}

// Tails of the plan tables and unfilled slots, spread over the whole grid.
__device__ __forceinline__ void plan_tails(const PlanShape &sh, const PlanPtrs &p,
                                           const int32_t *s_upre) {
    const int R = sh.R, SK = sh.SK;
    const int P = p.n_list[0];
    const int gt = blockIdx.x * kAssignThreads + threadIdx.x;
    const int gn = gridDim.x * kAssignThreads;
    const int sp = sh.G + sh.dcap + 1, se = sh.G + sh.dcap;
    const int ntab = R * sh.dcap;  // < 2^31: R, dcap <= 1024
    for (int x = gt; x < ntab; x += gn) {
        const int r = x / sh.dcap, j = x - r * sh.dcap;
        if (j >= p.n_dup[r]) {
            p.dup_expert[x] = -1;
            p.dup_start[x] = -1;
            p.dup_count[x] = 0;
            p.seg_ptr[(int64_t)r * sp + sh.G + 1 + j] = -1;
            p.seg_expert[(int64_t)r * se + sh.G + j] = -1;
        }
    }
    for (int x = P + gt; x < sh.pcap; x += gn) {
        p.list_expert[x] = -1;
        p.list_rank[x] = -1;
        p.list_b[x] = -1;
        p.piece_js[x] = -1;
    }
    // slots that receive nothing (only when some ids were dropped): the last
    // upre[r+1] - upre[r] slots of rank r
    const int n_empty = s_upre[R];
    for (int j = gt; j < n_empty; j += gn) {
        const int r2 = upper_bound(s_upre, R + 1, j) - 1;
        const int u = s_upre[r2 + 1] - s_upre[r2];
        p.src[(int64_t)r2 * SK + (SK - u) + (j - s_upre[r2])] = -1;
    }
}

// The assign passes over one tile, once its ids are in idv and the plan tables
// the placement needs are in regs (fetch_tables). by_tokens: K >= 4 and no
// repeated ids in the plan's status (else the bit-slice ranks). smem holds
// assign_lds_bytes().
__device__ __forceinline__ void assign_tile(const PlanShape &sh, const PlanPtrs &p, const Tile &t,
                                            const int (&idv)[kChunks], const TableRegs &regs,
                                            bool by_tokens, int32_t *smem) {
    uint32_t *s_pos = reinterpret_cast<uint32_t *>(smem);
    AsgTables tb;
    asg_tables(sh.E, sh.R, sh.pcap, tile_cap(sh), smem + pos_ints(sh), &tb);
    zero_pos(sh, s_pos);
    __syncthreads();
    int rank[kChunks];
    rank_entries(sh, idv, by_tokens, rank, s_pos);
    store_tables(sh, regs, tb);
    __syncthreads();
    // the tile's count of expert threadIdx.x -> where the expert starts in the list
    const int cnt = running_positions(sh, s_pos);
    int start, n_valid;
    block_excl_scan<1>(&cnt, &start, &n_valid, tb.scan_w);  // its barriers publish s_pos
    if ((int)threadIdx.x < sh.E) tb.toff[threadIdx.x] = start;
    __syncthreads();
    order_entries(sh, idv, rank, s_pos, tb);
    __syncthreads();
    int32_t *s_dst = reinterpret_cast<int32_t *>(s_pos);  // the counts are spent
    place_sorted(sh, p, t, n_valid, tb, s_dst);
    __syncthreads();
    write_dst(sh, p, t, idv, s_dst);
    plan_tails(sh, p, tb.upre);
}

// ---------------------------------------------------------------- k_assign
// Two 16-wave workgroups per CU need eight waves per SIMD; the attribute makes the
// compiler budget scalar registers for that (the plan pointers would otherwise
// hold enough of them to allow only one).
__global__ __launch_bounds__(kAssignThreads) __attribute__((amdgpu_waves_per_eu(8)))
void k_assign(const int32_t *__restrict__ ids, PlanShape sh, PlanPtrs) {
    extern __shared__ int32_t smem[];
    touch_kernargs<TileArgs>();
    const PlanPtrs &p = plan_ptrs<TileArgs>();
    const Tile t = tile_of(sh, blockIdx.x);
    // loads first, all in flight: the status, this wave's ids, then the tables,
    // which are only needed once the ranks are taken
    const int status = p.status[0];
    int idv[kChunks];
    load_ids(sh, ids, t, idv);
    const TableRegs regs = fetch_tables(sh, p, t.tile, true);
    assign_tile(sh, p, t, idv, regs, sh.K >= 4 && !(status & MOONEP_STATUS_REPEAT_ID), smem);
}

// ---------------------------------------------------------------- k_plan_fused
// The plan in two launches, for problems with few tiles (the decode shape):
// after k_count, one 1024-thread workgroup per tile
//   1. sums every tile's counts: T, and the counts of the tiles before its own
//      (its tile base), threads split as (tile group, expert) and the group
//      partials added in LDS;
//   2. runs the solve itself -- every workgroup the same deterministic solve on
//      the same T, so every workgroup writes the same values to the same plan
//      entries, and reads back only what it wrote itself (a workgroup barrier
//      makes its own global writes visible to all its threads);
//   3. assigns its tile as k_assign does.
// No workgroup waits for another, so nothing depends on which workgroups are
// resident at once. The cost is the redundant solve and the count reads, both
// small at the shapes that take this path (n_tiles * E bounded by kFusedMaxCounts).
// Te = T of expert threadIdx.x and base = its count in tiles before `tile` (both
// 0 beyond E), from the 16-bit counts k_count<..., true> wrote; s_part holds
// gather_part_bytes(). A load takes V consecutive counts: 8 (16 bytes) when
// E % 8 == 0, 2 when E is even, else 1 (rows of E counts are then aligned to the
// load). Threads split as (tile group, column of V experts): group g of `groups`
// takes tiles g, g + groups, ..., each thread keeping U loads in flight; the
// group partials are added in LDS.
constexpr int kGatherUnroll = 16;

// Counts per load: 8 (16 bytes) when E % 8 == 0, 2 when E is even, else 1.
__host__ __device__ inline int gather_width(int E) { return (E & 7) == 0 ? 8 : (E & 1) == 0 ? 2 : 1; }

// Tile groups of the gather: as many as the threads allow, but no more than one
// batch of `unroll` loads per thread needs (the partials are added serially).
__host__ __device__ inline int gather_groups(int n_tiles, int cols, int unroll) {
    const int most = kAssignThreads / cols;  // >= 1: cols <= E <= kAssignThreads
    const int need = (n_tiles + unroll - 1) / unroll;
    const int g = most < need ? most : need;
    return g > 1 ? g : 1;
}

// Unroll of the gather in each form of the fused kernel (the bounded solve leaves
// fewer registers to hold loads in flight) and the ints of its LDS partials.
template <bool BOUNDED>
constexpr int gather_unroll() { return BOUNDED ? kGatherUnroll / 2 : kGatherUnroll; }

inline size_t gather_part_bytes(const PlanShape &sh, bool bounded) {
    const int u = bounded ? gather_unroll<true>() : gather_unroll<false>();
    return sizeof(int32_t) * 2 * (size_t)sh.E *
           gather_groups(sh.n_tiles, sh.E / gather_width(sh.E), u);
}

template <int V>
struct Counts16;
template <>
struct Counts16<8> {
    typedef uint16_t type __attribute__((ext_vector_type(8)));
    __device__ static int at(const type &x, int v) { return x[v]; }
};
template <>
struct Counts16<2> {
    typedef uint16_t type __attribute__((ext_vector_type(2)));
    __device__ static int at(const type &x, int v) { return x[v]; }
};
template <>
struct Counts16<1> {
    typedef uint16_t type;
    __device__ static int at(const type &x, int) { return x; }
};

template <int V, int U>
__device__ __forceinline__ void gather_cols(const PlanShape &sh, const PlanPtrs &p, int tile,
                                            int *s_part) {
    typedef typename Counts16<V>::type vec_t;
    const int tid = threadIdx.x;
    const int cols = sh.E / V;
    const int groups = gather_groups(sh.n_tiles, cols, U);
    const int g = tid / cols, c = tid - g * cols;
    if (g >= groups) return;
    int sum[V], pre[V];
#pragma unroll
    for (int v = 0; v < V; ++v) sum[v] = pre[v] = 0;
    const vec_t *col = reinterpret_cast<const vec_t *>(p.tile_counts) + c;
    // one batch of loads from tiles u0, u0 + groups, ...; the first batch is
    // straight-line code, so that its loads issue together with the caller's
    // earlier ones (a loop header makes the compiler wait for those first)
    auto batch = [&](int u0) {
        vec_t x[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int u = u0 + j * groups;
            x[j] = u < sh.n_tiles ? col[(int64_t)u * cols] : vec_t{};
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const bool before = u0 + j * groups < tile;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int n = Counts16<V>::at(x[j], v);
                sum[v] += n;
                pre[v] += before ? n : 0;
            }
        }
    };
    batch(g);
    for (int u0 = g + groups * U; u0 < sh.n_tiles; u0 += groups * U) batch(u0);
#pragma unroll
    for (int v = 0; v < V; ++v) {
        s_part[g * sh.E + c * V + v] = sum[v];
        s_part[(groups + g) * sh.E + c * V + v] = pre[v];
    }
}

template <int U>
__device__ __forceinline__ void gather_counts(const PlanShape &sh, const PlanPtrs &p, int tile,
                                              int &Te, int &base, int *s_part) {
    const int tid = threadIdx.x;
    const int V = gather_width(sh.E);
    if (V == 8) gather_cols<8, U>(sh, p, tile, s_part);
    else if (V == 2) gather_cols<2, U>(sh, p, tile, s_part);
    else gather_cols<1, U>(sh, p, tile, s_part);
    const int groups = gather_groups(sh.n_tiles, sh.E / V, U);
    __syncthreads();
    Te = 0;
    base = 0;
    if (tid < sh.E) {
        for (int q = 0; q < groups; ++q) {
            Te += s_part[q * sh.E + tid];
            base += s_part[(groups + q) * sh.E + tid];
        }
    }
    __syncthreads();  // s_part is the solve's LDS next
}

template <bool BOUNDED>
__device__ __forceinline__ void plan_fused(const int32_t *__restrict__ ids, const PlanShape &sh,
                                           const PlanPtrs &p) {
    extern __shared__ int32_t smem[];
    const int tid = threadIdx.x;
    const Tile t = tile_of(sh, blockIdx.x);
    // the tiles' status words, (water-fill) this tile's ids and the counts
    // first, so that they share one round trip and the ids are in by the time
    // they are ranked; the bounded solve needs the registers the ids would hold
    // across it, so there they are loaded after the solve
    int st = tid < sh.n_tiles ? p.tile_status[tid] : 0;
    int idv[kChunks];
    if constexpr (!BOUNDED) load_ids(sh, ids, t, idv);
    int Te, base;
    gather_counts<gather_unroll<BOUNDED>()>(sh, p, t.tile, Te, base, smem);
    for (int u = tid + kAssignThreads; u < sh.n_tiles; u += kAssignThreads) st |= p.tile_status[u];
    if (blockIdx.x == 0 && tid < sh.E) p.T[tid] = Te;
    int status;
    if constexpr (BOUNDED) status = solve_bounded(sh, p, smem, Te, st);
    else status = solve_waterfill(sh, p, smem, Te, st);
    __syncthreads();  // this workgroup's plan writes are visible to all its threads
    if constexpr (BOUNDED) load_ids(sh, ids, t, idv);
    TableRegs regs = fetch_tables(sh, p, t.tile, false);
    regs.tbase = base;
    assign_tile(sh, p, t, idv, regs, sh.K >= 4 && !(status & MOONEP_STATUS_REPEAT_ID), smem);
}

template <bool BOUNDED>
__global__ __launch_bounds__(kAssignThreads) void k_plan_fused(const int32_t *__restrict__ ids,
                                                               PlanShape sh, PlanPtrs) {
    touch_kernargs<TileArgs>();
    plan_fused<BOUNDED>(ids, sh, plan_ptrs<TileArgs>());
}

constexpr size_t kMaxLdsBytes = 160 * 1024;  // LDS one workgroup may hold on gfx950

// Launches with more dynamic LDS than the default 64 KiB need the kernel's limit
// raised. It is raised once per kernel and device, to the whole kMaxLdsBytes,
// so that a plan call makes no attribute call after the first (the host's time
// between the plan's launches is time the device can sit idle).
enum LdsKernel { kLdsFusedBounded, kLdsFused, kLdsSolveBounded, kLdsSolve, kLdsAssign, kLdsKernels };
constexpr int kLdsDevices = 64;
std::atomic<uint8_t> g_lds_raised[kLdsDevices][kLdsKernels];

hipError_t allow_lds(const void *kernel, LdsKernel which, size_t lds) {
    if (lds <= 65536) return hipSuccess;  // within the default dynamic LDS limit of a launch
    if (lds > kMaxLdsBytes) return hipErrorInvalidValue;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < kLdsDevices;
    if (cached && g_lds_raised[dev][which].load(std::memory_order_acquire)) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLdsBytes);
    if (e == hipSuccess && cached) g_lds_raised[dev][which].store(1, std::memory_order_release);
    return e;
}

}  // namespace

hipError_t launch_plan(const PlanShape &sh, const int32_t *ids, const PlanPtrs &p, bool bounded,
                       hipStream_t st) {
    const dim3 tiles(sh.n_tiles);
#define MOONEP_COUNT(KM)                                                                      \
    do {                                                                                      \
        if (sh.launches == 2)                                                                 \
            hipLaunchKernelGGL((k_count<KM, true>), tiles, dim3(kPlanThreads), 0, st, ids,    \
                               sh, p.tile_counts, p.tile_status);                             \
        else                                                                                  \
            hipLaunchKernelGGL((k_count<KM, false>), tiles, dim3(kPlanThreads), 0, st, ids,   \
                               sh, p.tile_counts, p.tile_status);                             \
    } while (0)
    if (sh.K <= 1) MOONEP_COUNT(1);
    else if (sh.K <= 2) MOONEP_COUNT(2);
    else if (sh.K <= 4) MOONEP_COUNT(4);
    else if (sh.K <= 8) MOONEP_COUNT(8);
    else if (sh.K <= 16) MOONEP_COUNT(16);
    else if (sh.K <= 32) MOONEP_COUNT(32);
    else MOONEP_COUNT(64);
#undef MOONEP_COUNT
    if (sh.launches == 2) {
        // the gather's partials come first, then the solve's LDS, then assign's
        size_t lds = solve_lds_bytes(sh, bounded);
        lds = lds > assign_lds_bytes(sh) ? lds : assign_lds_bytes(sh);
        const size_t part = gather_part_bytes(sh, bounded);
        lds = lds > part ? lds : part;
        const void *k = bounded ? (const void *)k_plan_fused<true> : (const void *)k_plan_fused<false>;
        hipError_t e = allow_lds(k, bounded ? kLdsFusedBounded : kLdsFused, lds);
        if (e != hipSuccess) return e;
        if (bounded)
            hipLaunchKernelGGL(k_plan_fused<true>, tiles, dim3(kAssignThreads), lds, st, ids, sh, p);
        else
            hipLaunchKernelGGL(k_plan_fused<false>, tiles, dim3(kAssignThreads), lds, st, ids, sh, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_scan, dim3((sh.E + 63) / 64), dim3(kScanThreads), 0, st, sh,
                       p.tile_counts, p.T);
    const size_t slds = solve_lds_bytes(sh, bounded);
    hipError_t e = allow_lds(bounded ? (const void *)k_solve_bounded : (const void *)k_solve,
                             bounded ? kLdsSolveBounded : kLdsSolve, slds);
    if (e != hipSuccess) return e;
    if (bounded) hipLaunchKernelGGL(k_solve_bounded, dim3(1), dim3(kSolveThreads), slds, st, sh, p);
    else hipLaunchKernelGGL(k_solve, dim3(1), dim3(kSolveThreads), slds, st, sh, p);
    const size_t lds = assign_lds_bytes(sh);
    e = allow_lds((const void *)k_assign, kLdsAssign, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_assign, tiles, dim3(kAssignThreads), lds, st, ids, sh, p);
    return hipGetLastError();
}

}  // namespace moonep
