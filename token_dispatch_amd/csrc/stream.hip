// Streaming kernels for gfx950 that measure practical HBM ceilings (plain
// sequential read, write, copy). Not part of the method; see moonep_stream.h.
//
// Two launch shapes, chosen by the caller's chunk_bytes:
//   0      one resident grid (as many 256-thread workgroups as the device holds
//          at once) walks the buffer with a grid-stride loop;
//   c > 0  one workgroup per contiguous chunk of c bytes (the last one shorter),
//          so each workgroup streams through its own region.
// Every thread keeps kUnroll 16-byte accesses in flight per iteration,
// consecutive lanes on consecutive 16-byte chunks, so every wave-wide access is
// a 1 KiB burst.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moonep_stream.h"

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr uint32_t kSinkMagic = 0x9e3779b9u;

// The 16-byte chunks a workgroup walks: [first, n) in steps of `step` (grid
// stride), or its own chunk [first, end) in steps of one iteration's span.
struct Walk {
    int64_t first, end, step;
};

__device__ __forceinline__ Walk walk_of(int64_t n, int64_t chunk) {
    constexpr int64_t kSpan = (int64_t)kThreads * kUnroll;
    if (chunk == 0)
        return Walk{(int64_t)blockIdx.x * kSpan + threadIdx.x, n, (int64_t)gridDim.x * kSpan};
    const int64_t b = (int64_t)blockIdx.x * chunk;
    const int64_t e = b + chunk < n ? b + chunk : n;
    return Walk{b + threadIdx.x, e, kSpan};
}

__global__ __launch_bounds__(kThreads) void k_stream_read(const v4u *__restrict__ src, int64_t n,
                                                          int64_t chunk, v4u *__restrict__ sink) {
    const Walk wk = walk_of(n, chunk);
    const int64_t step = wk.step;
    n = wk.end;
    uint32_t acc = 0;
    for (int64_t base = wk.first; base < n; base += step) {
        v4u v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kThreads;
            v[u] = i < n ? __builtin_nontemporal_load(src + i) : v4u{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc = (acc ^ v[u].x ^ v[u].y ^ v[u].z ^ v[u].w) * 3u + 1u;
    }
    if (acc == kSinkMagic) *sink = v4u{acc, acc, acc, acc};
}

__global__ __launch_bounds__(kThreads) void k_stream_write(v4u *__restrict__ dst, int64_t n,
                                                           int64_t chunk, uint32_t pattern) {
    const Walk wk = walk_of(n, chunk);
    const int64_t step = wk.step;
    n = wk.end;
    const v4u p = v4u{pattern, pattern, pattern, pattern};
    for (int64_t base = wk.first; base < n; base += step) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kThreads;
            if (i < n) dst[i] = p;
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_stream_copy(v4u *__restrict__ dst,
                                                          const v4u *__restrict__ src, int64_t n,
                                                          int64_t chunk) {
    const Walk wk = walk_of(n, chunk);
    const int64_t step = wk.step;
    n = wk.end;
    for (int64_t base = wk.first; base < n; base += step) {
        v4u v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kThreads;
            if (i < n) v[u] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kThreads;
            if (i < n) dst[i] = v[u];
        }
    }
}

// Workgroups of `kernel` the current device holds at once (at least 1); not
// cached: these kernels are timed after warm-up calls.
template <typename F>
int64_t resident_grid(F kernel) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return (int64_t)cus * per_cu;
}

bool ok16(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workgroups of a launch over n 16-byte chunks: one resident grid (chunk16 == 0,
// no more workgroups than iterations), or one per chunk of chunk16 16-byte units.
int64_t grid_for(int64_t n, int64_t chunk16, int64_t resident) {
    if (chunk16 > 0) return (n + chunk16 - 1) / chunk16;
    const int64_t need = (n + kThreads * kUnroll - 1) / (kThreads * kUnroll);
    return need < resident ? need : resident;
}

// chunk_bytes: 0, or a positive multiple of 4096 whose workgroup count fits a
// grid dimension.
bool chunk_ok(int64_t bytes, int64_t chunk_bytes) {
    if (chunk_bytes == 0) return true;
    if (chunk_bytes < 0 || chunk_bytes % 4096 != 0) return false;
    return (bytes + chunk_bytes - 1) / chunk_bytes < ((int64_t)1 << 31);
}

}  // namespace

extern "C" {

int moonep_stream_read(const void *src, int64_t bytes, int64_t chunk_bytes, void *sink,
                       void *stream) {
    if (bytes <= 0 || bytes % 16 != 0 || !chunk_ok(bytes, chunk_bytes)) return -1;
    if (!ok16(src) || !ok16(sink)) return -2;
    const int64_t n = bytes / 16, c = chunk_bytes / 16;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_stream_read,
                       dim3((unsigned)grid_for(n, c, c ? 0 : resident_grid(k_stream_read))),
                       dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const v4u *>(src), n, c, static_cast<v4u *>(sink));
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

int moonep_stream_write(void *dst, int64_t bytes, int64_t chunk_bytes, uint32_t pattern,
                        void *stream) {
    if (bytes <= 0 || bytes % 16 != 0 || !chunk_ok(bytes, chunk_bytes)) return -1;
    if (!ok16(dst)) return -2;
    const int64_t n = bytes / 16, c = chunk_bytes / 16;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_stream_write,
                       dim3((unsigned)grid_for(n, c, c ? 0 : resident_grid(k_stream_write))),
                       dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<v4u *>(dst), n, c, pattern);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

int moonep_stream_copy(void *dst, const void *src, int64_t bytes, int64_t chunk_bytes,
                       void *stream) {
    if (bytes <= 0 || bytes % 16 != 0 || !chunk_ok(bytes, chunk_bytes)) return -1;
    if (!ok16(dst) || !ok16(src)) return -2;
    const int64_t n = bytes / 16, c = chunk_bytes / 16;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_stream_copy,
                       dim3((unsigned)grid_for(n, c, c ? 0 : resident_grid(k_stream_copy))),
                       dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<v4u *>(dst), static_cast<const v4u *>(src), n, c);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
