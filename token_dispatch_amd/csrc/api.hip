// C-ABI entry points: argument checks, the plan-buffer layout, and kernel
// launches on the caller's stream. No call allocates, frees or synchronises.
#include <string.h>

#include <atomic>
#include <mutex>

#include "internal.h"

// The plan kernels' scratch for moonep_plan_noscratch: one array per GPU in the
// library's device memory, held from the first use on a GPU until the process
// ends. In host code the name is only a stand-in, never a device address: the
// address is looked up once per device (static_scratch below) and that pointer
// is what the kernels get.
static __device__ __align__(256) unsigned char scratch[MOONEP_STATIC_SCRATCH_BYTES];

namespace moonep {
namespace {

constexpr int64_t kAlign = 256;

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int elem_bytes(int32_t dtype) { return dtype == MOONEP_BF16 ? 2 : 4; }

bool aligned16(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims(const moonep_dims *d) {
    if (d == nullptr) return MOONEP_ERR_PTR;
    if (d->R < 1 || d->R > kMaxR) return MOONEP_ERR_DIMS;
    if (d->E < d->R || d->E > kMaxE || d->E % d->R != 0) return MOONEP_ERR_DIMS;
    if (d->K < 1 || d->K > d->E || d->K > kMaxK) return MOONEP_ERR_DIMS;
    if (d->S < 1 || d->B < 0) return MOONEP_ERR_DIMS;
    if ((int64_t)d->R * d->S * d->K >= ((int64_t)1 << 31)) return MOONEP_ERR_DIMS;
    if (d->dtype != MOONEP_F32 && d->dtype != MOONEP_BF16) return MOONEP_ERR_DIMS;
    const int64_t row = (int64_t)d->H * elem_bytes(d->dtype);
    if (d->H < 1 || row % 16 != 0) return MOONEP_ERR_DIMS;
    // 16-byte chunks of one row are indexed with int32 inside the kernels
    if (row / 16 >= ((int64_t)1 << 31)) return MOONEP_ERR_DIMS;
    return MOONEP_OK;
}

PlanShape shape_of(const moonep_dims *d, const moonep_layout &lay) {
    PlanShape s;
    s.R = d->R;
    s.E = d->E;
    s.K = d->K;
    s.S = d->S;
    s.B = d->B;
    s.G = d->E / d->R;
    s.SK = d->S * d->K;
    s.n_tok = d->R * d->S;
    s.n_ent = d->R * d->S * d->K;
    s.dcap = lay.dcap;
    s.pcap = lay.pcap;
    s.n_tiles = lay.n_tiles;
    s.tile_tokens = lay.tile_tokens;
    s.tile_chunks = (lay.tile_tokens * d->K + 1023) / 1024;
    int bits = 0;
    while ((1 << bits) < d->E) ++bits;
    s.id_bits = bits;
    s.inv_k = 1.0f / (float)d->K;
    s.launches = lay.plan_launches;
    return s;
}

int launch_rc(hipError_t e) { return e == hipSuccess ? MOONEP_OK : MOONEP_ERR_HIP; }

// Device address of `scratch` on the current device, looked up with
// hipGetSymbolAddress on the first call made with that device current and kept.
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int static_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOONEP_ERR_HIP;
    void *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (ptr == nullptr) {
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
                (void)hipGetLastError();
                return MOONEP_ERR_HIP;
            }
            g_scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return MOONEP_OK;
}

}  // namespace

PlanPtrs resolve(const moonep_layout &l, void *base) {
    return resolve(l, base, static_cast<char *>(base) + l.persist_bytes);
}

PlanPtrs resolve(const moonep_layout &l, void *base, void *scratch_base) {
    auto at = [base](int64_t off) { return reinterpret_cast<int32_t *>(static_cast<char *>(base) + off); };
    // offsets at or past persist_bytes are taken from scratch_base instead
    auto sc = [&l, scratch_base](int64_t off) {
        return reinterpret_cast<int32_t *>(static_cast<char *>(scratch_base) + (off - l.persist_bytes));
    };
    PlanPtrs p;
    p.status = at(l.status);
    p.maxT = at(l.maxT);
    p.maxvio = reinterpret_cast<double *>(static_cast<char *>(base) + l.maxvio);
    p.T = at(l.T);
    p.hoff = at(l.hoff);
    p.L = at(l.L);
    p.keep = at(l.keep);
    p.O = at(l.O);
    p.D = at(l.D);
    p.Opre = at(l.Opre);
    p.Dpre = at(l.Dpre);
    p.dst = at(l.dst);
    p.src = at(l.src);
    p.n_dup = at(l.n_dup);
    p.dup_expert = at(l.dup_expert);
    p.dup_start = at(l.dup_start);
    p.dup_count = at(l.dup_count);
    p.seg_ptr = at(l.seg_ptr);
    p.seg_expert = at(l.seg_expert);
    p.n_list = at(l.n_list);
    p.list_expert = at(l.list_expert);
    p.list_rank = at(l.list_rank);
    p.list_b = at(l.list_b);
    p.dup_ptr = at(l.dup_ptr);
    p.mat_pre = at(l.ws_mat_pre);
    p.xlist = at(l.ws_xlist);
    p.n_x = at(l.ws_n_x);
    p.tile_counts = sc(l.ws_tile_counts);
    p.tile_status = sc(l.ws_tile_status);
    p.piece_js = sc(l.ws_piece_js);
    p.kept = sc(l.ws_kept);
    p.koff = sc(l.ws_koff);
    p.upre = sc(l.ws_upre);
    p.pslot = sc(l.ws_pslot);
    p.pcnt = sc(l.ws_pcnt);
    return p;
}

}  // namespace moonep

using namespace moonep;

extern "C" {

int moonep_plan_layout(const moonep_dims *d, moonep_layout *out) {
    if (out == nullptr) return MOONEP_ERR_PTR;
    const int rc = check_dims(d);
    if (rc != MOONEP_OK) return rc;
    moonep_layout l;
    memset(&l, 0, sizeof(l));
    const int64_t R = d->R, E = d->E, G = E / R, SK = (int64_t)d->S * d->K;
    const int64_t NE = R * SK, n_tok = R * d->S;
    int64_t dcap = SK < E - G ? SK : E - G;
    if (dcap < 1) dcap = 1;
    l.dcap = (int32_t)dcap;
    l.pcap = (int32_t)(E + R);
    // Two launches when a tile of 1024, 2048 or 4096 entries keeps the counts that
    // every workgroup of the fused kernel reads (n_tiles * E) within
    // kFusedMaxCounts: the smallest such tile. Else four launches with the largest
    // tile that still gives kTileTarget tiles, so that small problems spread over
    // more of the device.
    auto tiles_of = [&](int64_t entries) {
        const int64_t tt = entries / d->K;
        return (n_tok + tt - 1) / tt;
    };
    int64_t tile_entries = 0;
    for (int64_t te = kMinTileEntries; te <= kTileEntries; te *= 2)
        if (tiles_of(te) * E <= kFusedMaxCounts) {
            tile_entries = te;
            break;
        }
    l.plan_launches = tile_entries > 0 ? 2 : 4;
    if (tile_entries == 0) {
        tile_entries = kTileEntries;
        while (tile_entries > kMinTileEntries && NE / tile_entries < kTileTarget) tile_entries /= 2;
    }
    l.tile_tokens = (int32_t)(tile_entries / d->K);
    l.n_tiles = (int32_t)tiles_of(tile_entries);
    int64_t off = 0;
    auto take = [&off](int64_t bytes) {
        const int64_t o = off;
        off = round_up(off + bytes, kAlign);
        return o;
    };
    l.status = take(4);
    l.maxT = take(4);
    l.maxvio = take(8);
    l.T = take(4 * E);
    l.hoff = take(4 * E);
    l.L = take(4 * R);
    l.keep = take(4 * R);
    l.O = take(4 * R);
    l.D = take(4 * R);
    l.Opre = take(4 * (R + 1));
    l.Dpre = take(4 * (R + 1));
    l.dst = take(4 * NE);
    l.src = take(4 * NE);
    l.n_dup = take(4 * R);
    l.dup_expert = take(4 * R * dcap);
    l.dup_start = take(4 * R * dcap);
    l.dup_count = take(4 * R * dcap);
    l.seg_ptr = take(4 * R * (G + dcap + 1));
    l.seg_expert = take(4 * R * (G + dcap));
    l.n_list = take(4);
    l.list_expert = take(4 * (int64_t)l.pcap);
    l.list_rank = take(4 * (int64_t)l.pcap);
    l.list_b = take(4 * (int64_t)l.pcap);
    l.dup_ptr = take(4 * (E + 1));
    // workspace that later calls read (replicate: mat_pre; reduce: xlist, n_x)
    l.ws_mat_pre = take(4 * (R + 1));
    l.ws_xlist = take(4 * E);
    l.ws_n_x = take(4);
    l.persist_bytes = off;
    // scratch of the plan kernels alone, last, so that it can live elsewhere
    l.ws_tile_counts = take(4 * (int64_t)l.n_tiles * E);
    l.ws_tile_status = take(4 * (int64_t)l.n_tiles);
    l.ws_piece_js = take(4 * (int64_t)l.pcap);
    l.ws_kept = take(4 * E);
    l.ws_koff = take(4 * E);
    l.ws_upre = take(4 * (R + 1));
    l.ws_pslot = take(4 * (int64_t)l.pcap);
    l.ws_pcnt = take(4 * (int64_t)l.pcap);
    l.bytes = off;
    *out = l;
    return MOONEP_OK;
}

int moonep_plan_ex(const moonep_dims *d, const int32_t *topk_ids, void *plan_buf, int32_t flags,
                   void *stream) {
    moonep_layout l;
    int rc = moonep_plan_layout(d, &l);
    if (rc != MOONEP_OK) return rc;
    const int32_t known = MOONEP_PLAN_BOUNDED | MOONEP_PLAN_FOUR_LAUNCH | MOONEP_PLAN_TWO_LAUNCH;
    if ((flags & ~known) != 0 ||
        ((flags & MOONEP_PLAN_FOUR_LAUNCH) && (flags & MOONEP_PLAN_TWO_LAUNCH)))
        return MOONEP_ERR_DIMS;
    if (!aligned16(topk_ids) || !aligned16(plan_buf)) return MOONEP_ERR_PTR;
    PlanShape sh = shape_of(d, l);
    if (flags & MOONEP_PLAN_FOUR_LAUNCH) sh.launches = 4;
    if (flags & MOONEP_PLAN_TWO_LAUNCH) sh.launches = 2;
    (void)hipGetLastError();
    return launch_rc(launch_plan(sh, topk_ids, resolve(l, plan_buf),
                                 (flags & MOONEP_PLAN_BOUNDED) != 0,
                                 static_cast<hipStream_t>(stream)));
}

int moonep_plan(const moonep_dims *d, const int32_t *topk_ids, void *plan_buf, void *stream) {
    return moonep_plan_ex(d, topk_ids, plan_buf, 0, stream);
}

int moonep_plan_bounded(const moonep_dims *d, const int32_t *topk_ids, void *plan_buf,
                        void *stream) {
    return moonep_plan_ex(d, topk_ids, plan_buf, MOONEP_PLAN_BOUNDED, stream);
}

int moonep_plan_noscratch(const moonep_dims *d, const int32_t *topk_ids, void *plan_buf,
                          int32_t bounded, void *stream) {
    moonep_layout l;
    int rc = moonep_plan_layout(d, &l);
    if (rc != MOONEP_OK) return rc;
    if (bounded != 0 && bounded != 1) return MOONEP_ERR_DIMS;
    if (!aligned16(topk_ids) || !aligned16(plan_buf)) return MOONEP_ERR_PTR;
    if (l.bytes - l.persist_bytes > (int64_t)MOONEP_STATIC_SCRATCH_BYTES) return MOONEP_ERR_SIZE;
    void *scr = nullptr;
    rc = static_scratch(&scr);
    if (rc != MOONEP_OK) return rc;
    const PlanShape sh = shape_of(d, l);
    (void)hipGetLastError();
    return launch_rc(launch_plan(sh, topk_ids, resolve(l, plan_buf, scr), bounded != 0,
                                 static_cast<hipStream_t>(stream)));
}

int moonep_dispatch(const moonep_dims *d, const void *plan_buf, const void *hidden, void *recv,
                    void *stream) {
    moonep_layout l;
    int rc = moonep_plan_layout(d, &l);
    if (rc != MOONEP_OK) return rc;
    if (!aligned16(plan_buf) || !aligned16(hidden) || !aligned16(recv)) return MOONEP_ERR_PTR;
    const PlanShape sh = shape_of(d, l);
    (void)hipGetLastError();
    return launch_rc(launch_dispatch(sh, resolve(l, const_cast<void *>(plan_buf)), hidden,
                                     recv, d->H * elem_bytes(d->dtype),
                                     static_cast<hipStream_t>(stream)));
}

int moonep_replicate(const moonep_dims *d, const void *plan_buf, const void *expert_w,
                     void *dup_w, int64_t block_bytes, void *stream) {
    moonep_layout l;
    int rc = moonep_plan_layout(d, &l);
    if (rc != MOONEP_OK) return rc;
    if (block_bytes <= 0 || block_bytes % 16 != 0) return MOONEP_ERR_SIZE;
    if (d->B == 0) return MOONEP_OK;  // no duplicate slots: nothing to copy
    if (!aligned16(plan_buf) || !aligned16(expert_w) || !aligned16(dup_w)) return MOONEP_ERR_PTR;
    const PlanShape sh = shape_of(d, l);
    (void)hipGetLastError();
    return launch_rc(launch_replicate(sh, resolve(l, const_cast<void *>(plan_buf)), expert_w,
                                      dup_w, block_bytes, static_cast<hipStream_t>(stream)));
}

int moonep_combine(const moonep_dims *d, const void *plan_buf, const void *y, const float *topk_w,
                   void *out, int32_t out_dtype, void *stream) {
    moonep_layout l;
    int rc = moonep_plan_layout(d, &l);
    if (rc != MOONEP_OK) return rc;
    if (out_dtype != MOONEP_F32 && out_dtype != MOONEP_BF16) return MOONEP_ERR_DIMS;
    if (!aligned16(plan_buf) || !aligned16(y) || !aligned16(topk_w) || !aligned16(out))
        return MOONEP_ERR_PTR;
    const PlanShape sh = shape_of(d, l);
    (void)hipGetLastError();
    return launch_rc(launch_combine(sh, resolve(l, const_cast<void *>(plan_buf)), y, topk_w, out,
                                    d->dtype == MOONEP_BF16, out_dtype == MOONEP_BF16, d->H,
                                    static_cast<hipStream_t>(stream)));
}

int moonep_reduce_dup_grads(const moonep_dims *d, const void *plan_buf, const float *dup_grads,
                            float *home_grads, int64_t block_elems, void *stream) {
    moonep_layout l;
    int rc = moonep_plan_layout(d, &l);
    if (rc != MOONEP_OK) return rc;
    if (block_elems <= 0 || block_elems % 4 != 0) return MOONEP_ERR_SIZE;
    if (d->B == 0) return MOONEP_OK;  // no duplicate slots: nothing to add
    if (!aligned16(plan_buf) || !aligned16(dup_grads) || !aligned16(home_grads))
        return MOONEP_ERR_PTR;
    const PlanShape sh = shape_of(d, l);
    (void)hipGetLastError();
    return launch_rc(launch_reduce(sh, resolve(l, const_cast<void *>(plan_buf)), dup_grads,
                                   home_grads, block_elems, static_cast<hipStream_t>(stream)));
}

int moonep_combine_backward(const moonep_dims *d, const void *plan_buf, const void *grad_out,
                            int32_t gout_dtype, const float *topk_w, const void *y, void *grad_y,
                            float *grad_w, void *stream) {
    moonep_layout l;
    int rc = moonep_plan_layout(d, &l);
    if (rc != MOONEP_OK) return rc;
    if (gout_dtype != MOONEP_F32 && gout_dtype != MOONEP_BF16) return MOONEP_ERR_DIMS;
    // grad_out rows must also split into 16-byte chunks
    if (((int64_t)d->H * elem_bytes(gout_dtype)) % 16 != 0) return MOONEP_ERR_DIMS;
    if (grad_y == nullptr && grad_w == nullptr) return MOONEP_OK;  // nothing asked for
    if (!aligned16(plan_buf) || !aligned16(grad_out)) return MOONEP_ERR_PTR;
    if (grad_y != nullptr && (!aligned16(grad_y) || !aligned16(topk_w))) return MOONEP_ERR_PTR;
    if (grad_w != nullptr && (!aligned16(grad_w) || !aligned16(y))) return MOONEP_ERR_PTR;
    const PlanShape sh = shape_of(d, l);
    (void)hipGetLastError();
    return launch_rc(launch_combine_backward(sh, resolve(l, const_cast<void *>(plan_buf)), grad_out,
                                             gout_dtype == MOONEP_BF16, topk_w, y, grad_y, grad_w,
                                             d->dtype == MOONEP_BF16, d->H,
                                             static_cast<hipStream_t>(stream)));
}

int moonep_dispatch_backward(const moonep_dims *d, const void *plan_buf, const void *grad_recv,
                             void *grad_hidden, int32_t out_dtype, void *stream) {
    moonep_layout l;
    int rc = moonep_plan_layout(d, &l);
    if (rc != MOONEP_OK) return rc;
    if (out_dtype != MOONEP_F32 && out_dtype != MOONEP_BF16) return MOONEP_ERR_DIMS;
    if (!aligned16(plan_buf) || !aligned16(grad_recv) || !aligned16(grad_hidden))
        return MOONEP_ERR_PTR;
    const PlanShape sh = shape_of(d, l);
    (void)hipGetLastError();
    return launch_rc(launch_dispatch_backward(sh, resolve(l, const_cast<void *>(plan_buf)),
                                              grad_recv, grad_hidden, d->dtype == MOONEP_BF16,
                                              out_dtype == MOONEP_BF16, d->H,
                                              static_cast<hipStream_t>(stream)));
}

int moonep_launch_count(const moonep_dims *d, int32_t op, int32_t *n_launches) {
    if (n_launches == nullptr) return MOONEP_ERR_PTR;
    moonep_layout l;
    const int rc = moonep_plan_layout(d, &l);
    if (rc != MOONEP_OK) return rc;
    if (op != MOONEP_OP_DISPATCH && op != MOONEP_OP_COMBINE) return MOONEP_ERR_DIMS;
    const PlanShape sh = shape_of(d, l);
    // the launchers only count while t_count_launches is set: no pointer is used
    const PlanPtrs p{};
    int32_t n = 0;
    t_count_launches = &n;
    const hipError_t e =
        op == MOONEP_OP_DISPATCH
            ? launch_dispatch(sh, p, nullptr, nullptr, d->H * elem_bytes(d->dtype), nullptr)
            : launch_combine(sh, p, nullptr, nullptr, nullptr, d->dtype == MOONEP_BF16,
                             d->dtype == MOONEP_BF16, d->H, nullptr);
    t_count_launches = nullptr;
    if (e != hipSuccess) return MOONEP_ERR_HIP;
    *n_launches = n;
    return MOONEP_OK;
}

const char *moonep_strerror(int rc) {
    switch (rc) {
        case MOONEP_OK: return "ok";
        case MOONEP_ERR_DIMS: return "invalid dims (range, divisibility or row alignment)";
        case MOONEP_ERR_PTR: return "NULL or misaligned (not 16-byte) pointer";
        case MOONEP_ERR_HIP: return "HIP kernel launch failed";
        case MOONEP_ERR_SIZE: return "inconsistent block size argument";
        default: return "unknown error";
    }
}

}  // extern "C"
