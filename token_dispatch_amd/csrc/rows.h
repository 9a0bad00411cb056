// Building blocks of the row-move kernels (move.hip, backward.hip): 16-byte
// vector types, lane utilities, bf16 rounding, the unpack of one 16-byte chunk
// of a row into binary32 values, the store of N results, and the host-side
// choice of chunks per lane and of the resident grid. Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moonep {
namespace rows {

// Native vectors: what global_load/store_dwordx{2,4} move, and what the
// non-temporal builtins accept.
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kMoveThreads = 256;
constexpr int kMoveWaves = kMoveThreads / 64;

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float readlane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two binary32 values rounded to bf16 (nearest even; a NaN stays a NaN of the
// same sign with its quiet bit set), a in the low half. This is one
// v_cvt_pk_bf16_f32 on gfx950, which rounds exactly like the bit-level rule
// (add 0x7fff plus the lowest kept bit, keep the top 16 bits; NaN: keep the top
// 16 bits and set bit 6).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}

// Rows read through a buffer resource: the row's base address and length sit in
// scalar registers and each lane only supplies a 32-bit byte offset, so a row
// load needs no 64-bit address arithmetic per lane. Offsets at or past the
// length read 0 (the hardware range check). A row qualifies when every lane's
// byte offset, including the lanes past the row's end in its last segment (at
// most 64 * 16 chunks further), stays below 2^31.
constexpr int64_t kBufRowChunks = (((int64_t)1 << 31) - ((int64_t)1 << 16)) / 16;
constexpr int kWordFormat = 0x00020000;  // raw (untyped) buffer of 32-bit words
constexpr int kPolicyNT = 2;             // non-temporal: each byte is read once

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const v4u *row, int32_t chunks) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<v4u *>(row), (short)0, chunks * 16,
                                             kWordFormat);
}

__device__ __forceinline__ v4u load_chunk_nt(__amdgpu_buffer_rsrc_t rs, int c) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, c * 16, 0, kPolicyNT);
}

// One 16-byte chunk of a row as binary32 values: 8 bf16 or 4 f32.
template <bool IN_BF16>
struct Chunk;
template <>
struct Chunk<true> {
    static constexpr int N = 8;
    __device__ static void unpack(const v4u &q, float *x) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float(w[j] << 16);
            x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    }
};
template <>
struct Chunk<false> {
    static constexpr int N = 4;
    __device__ static void unpack(const v4u &q, float *x) {
        x[0] = __uint_as_float(q.x);
        x[1] = __uint_as_float(q.y);
        x[2] = __uint_as_float(q.z);
        x[3] = __uint_as_float(q.w);
    }
};

// Store N binary32 results as elements elem0 .. elem0+N-1 of out (bf16: nearest
// even), non-temporally when NT.
template <bool NT, typename V>
__device__ __forceinline__ void put(V v, V *p) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <int N, bool OUT_BF16, bool NT>
__device__ __forceinline__ void store_elems(void *out, int64_t elem0, const float *a) {
    if constexpr (OUT_BF16) {
        uint32_t w[N / 2];
#pragma unroll
        for (int j = 0; j < N / 2; ++j) w[j] = pack_bf16x2(a[2 * j], a[2 * j + 1]);
        uint16_t *o = reinterpret_cast<uint16_t *>(out) + elem0;
        if constexpr (N == 8) {
            put<NT>(v4u{w[0], w[1], w[2], w[3]}, reinterpret_cast<v4u *>(o));
        } else {
            put<NT>(v2u{w[0], w[1]}, reinterpret_cast<v2u *>(o));
        }
    } else {
        float *o = reinterpret_cast<float *>(out) + elem0;
#pragma unroll
        for (int j = 0; j < N; j += 4)
            put<NT>(v4f{a[j], a[j + 1], a[j + 2], a[j + 3]}, reinterpret_cast<v4f *>(o + j));
    }
}

// Chunks per lane of one row segment: the row is split into the fewest segments
// of at most 16 chunks per lane, then each segment takes an instantiated width.
inline int pick_cpl(int64_t C) {
    const int64_t per_lane = (C + 63) / 64;
    const int64_t segs = (per_lane + 15) / 16;
    const int64_t need = (per_lane + segs - 1) / segs;
    static const int widths[] = {1, 2, 4, 7, 8, 14, 16};
    for (int w : widths)
        if (w >= need) return w;
    return 16;
}

// Row segments one wave of a rows-first kernel holds: as many as fit in about
// 200 VGPRs of row data, which keeps two waves per SIMD resident.
constexpr int tpw_of(int cpl) { return cpl >= 14 ? 3 : cpl >= 8 ? 6 : cpl >= 7 ? 7 : 8; }

// The same for kernels that also scale each copy (one segment fewer's worth of
// registers goes to the scaled values).
constexpr int scaled_tpw_of(int cpl) { return cpl >= 14 ? 2 : cpl >= 8 ? 4 : cpl >= 7 ? 5 : 6; }

// Workgroups of `kernel` (kMoveThreads each) the current device holds at once;
// `cache` is one int per device owned by the caller (0 = not yet queried; racing
// first calls store the same value).
template <typename F>
int resident_wgs(F kernel, int *cache) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (v > 0) return v;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kMoveThreads, 0) !=
            hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    v = cus * per_cu;
    __atomic_store_n(&cache[dev], v, __ATOMIC_RELAXED);
    return v;
}

}  // namespace rows
}  // namespace moonep
