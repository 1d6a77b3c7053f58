// gdn_device.hpp -- device helpers shared by the libgdn kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// Storage tags: the kernels are templated on these; values are always widened to fp32.
struct F32 {
    using storage = float;
    static constexpr int code = GDN_F32;
};
struct BF16 {
    using storage = uint16_t;
    static constexpr int code = GDN_BF16;
};
struct F16 {
    using storage = uint16_t;
    static constexpr int code = GDN_F16;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even (v_cvt on gfx950)
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);  // round to nearest even
}

template <typename T>
__device__ __forceinline__ float to_f32(typename T::storage v);
template <>
__device__ __forceinline__ float to_f32<F32>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<BF16>(uint16_t v) { return bf16_bits_to_f32(v); }
template <>
__device__ __forceinline__ float to_f32<F16>(uint16_t v) { return f16_bits_to_f32(v); }

template <typename T>
__device__ __forceinline__ typename T::storage from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<F32>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t from_f32<BF16>(float v) { return f32_to_bf16_bits(v); }
template <>
__device__ __forceinline__ uint16_t from_f32<F16>(float v) { return f32_to_f16_bits(v); }

// Load one element of a runtime-typed tensor (gate inputs) as fp32.
__device__ __forceinline__ float load_any(const void* p, int dtype, size_t i) {
    if (dtype == GDN_F32) return static_cast<const float*>(p)[i];
    const uint16_t h = static_cast<const uint16_t*>(p)[i];
    return dtype == GDN_BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
}

// Load 4 consecutive elements (8- or 16-byte aligned) and widen to fp32.
template <typename T>
__device__ __forceinline__ f32x4 load4(const typename T::storage* p);
template <>
__device__ __forceinline__ f32x4 load4<F32>(const float* p) {
    return *reinterpret_cast<const f32x4*>(p);
}
template <>
__device__ __forceinline__ f32x4 load4<BF16>(const uint16_t* p) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                 __uint_as_float(w.y & 0xffff0000u)};
}
template <>
__device__ __forceinline__ f32x4 load4<F16>(const uint16_t* p) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    return f32x4{f16_bits_to_f32(w.x & 0xffffu), f16_bits_to_f32(w.x >> 16), f16_bits_to_f32(w.y & 0xffffu),
                 f16_bits_to_f32(w.y >> 16)};
}

// Slices of K-wide rows (state columns, q/k rows) for kernels compiled for a width KP >= K.
// KX: K == KP, plain 16-byte (or 8-byte) accesses.  Otherwise elements at or past Kr read as zero
// and are not written, element by element (rows of any width and 4-byte alignment).
template <bool KX, bool NT>
__device__ __forceinline__ f32x4 ld_row4(const float* row, int e0, int Kr) {
    if constexpr (KX) {
        if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + e0));
        else return *reinterpret_cast<const f32x4*>(row + e0);
    } else {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = e0 + e < Kr ? row[e0 + e] : 0.0f;
        return r;
    }
}
template <bool KX, bool NT>
__device__ __forceinline__ void st_row4(float* row, int e0, int Kr, f32x4 v) {
    if constexpr (KX) {
        if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(row + e0));
        else *reinterpret_cast<f32x4*>(row + e0) = v;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e0 + e < Kr) row[e0 + e] = v[e];
    }
}
template <typename T, bool KX>
__device__ __forceinline__ f32x4 ld_in4(const typename T::storage* row, int e0, int Kr) {
    if constexpr (KX) {
        return load4<T>(row + e0);
    } else {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = e0 + e < Kr ? to_f32<T>(row[e0 + e]) : 0.0f;
        return r;
    }
}
// 16 raw bytes (VEC elements of type TS) of a row from element e0, elements at or past Kr zero.
template <typename TS, int VEC, bool KX>
__device__ __forceinline__ u32x4 ld_raw16(const TS* row, int e0, int Kr) {
    static_assert(VEC * sizeof(TS) == 16, "16 bytes");
    if constexpr (KX) {
        return *reinterpret_cast<const u32x4*>(row + e0);
    } else {
        union {
            u32x4 v;
            TS e[VEC];
        } u;
        u.v = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            if (e0 + e < Kr) u.e[e] = row[e0 + e];
        return u.v;
    }
}
// Compiled key width for a row width K <= 256: the next of 32, 64, 128, 256.
constexpr int padded_key_width(int K) { return K <= 32 ? 32 : K <= 64 ? 64 : K <= 128 ? 128 : 256; }

// DPP lane permutation of a float within rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <-> 7-i within each half row
constexpr int DPP_MIRROR = 0x140;     // lane i <-> 15-i within each row

// Sum over aligned groups of N consecutive lanes (N a power of two <= 64); every lane of a group
// receives the group's sum.  Within a 16-lane row the butterfly uses DPP; wider groups add
// cross-row swizzles.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (N >= 2) x += dpp<DPP_QUAD_XOR1>(x);
    if constexpr (N >= 4) x += dpp<DPP_QUAD_XOR2>(x);
    if constexpr (N >= 8) x += dpp<DPP_HALF_MIRROR>(x);
    if constexpr (N >= 16) x += dpp<DPP_MIRROR>(x);
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    if constexpr (N >= 64) x += __shfl_xor(x, 32);
    return x;
}

// Whole-call offsets check, done cooperatively by every thread of a block.  Offsets are valid iff
// offsets[0] == 0, offsets[B] == N and they never decrease (which keeps every entry in [0, N]).
// Must be reached by all threads of the block.  Returns true when the offsets are malformed.
__device__ __forceinline__ bool offsets_malformed(const int32_t* __restrict__ offsets, int B, int N) {
    int bad = 0;
    for (int i = threadIdx.x; i <= B; i += blockDim.x) {
        const int o = offsets[i];
        if (i == 0) bad |= (o != 0);
        else bad |= (offsets[i - 1] > o);
        if (i == B) bad |= (o != N);
    }
    return __syncthreads_or(bad) != 0;
}

// The block with linear index 0 reports the verdict of the offsets check.
__device__ __forceinline__ void report_status(int32_t* dev_status, bool malformed) {
    if (dev_status != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
        *dev_status = malformed ? GDN_ERR_OFFSETS : GDN_OK;
}

// Four consecutive gate inputs (element type T, the qkv type, or fp32), widened to fp32.
template <typename T>
__device__ __forceinline__ f32x4 load4_gate(const void* p, int gate_dtype, size_t i) {
    if (gate_dtype == GDN_F32) return load4<F32>(static_cast<const float*>(p) + i);
    return load4<T>(static_cast<const typename T::storage*>(p) + i);
}

// Tokens of a sequence of length len recorded by a capture of cap slots: min(counts[b], cap, len),
// at least 0, and 0 when the device flag active is given and reads 0.
__device__ __forceinline__ int captured_tokens(const int32_t* counts, const int32_t* active, int cap, int b,
                                               int len) {
    if (active != nullptr && active[0] == 0) return 0;
    int n = counts[b];
    n = n < cap ? n : cap;
    n = n < len ? n : len;
    return n > 0 ? n : 0;
}

// The capture record of one sequence (paged_ssm.rs page, DELTA_CAPTURE_INIT / _STEP): the row
// [cap*H decays | cap*HQ*K normalised keys | cap*H*V written values delta] of the fp32 capsule
// [B, cap*(H + HQ*K + H*V)].  Slot i holds token start + i.
struct CaptureRow {
    float* base;
    int cap, H, HQ, K, V;
    __device__ __forceinline__ float* g(int i, int h) const { return base + (size_t)i * H + h; }
    __device__ __forceinline__ float* k(int i, int kh) const {
        return base + (size_t)cap * H + ((size_t)i * HQ + kh) * K;
    }
    __device__ __forceinline__ float* d(int i, int h) const {
        return base + (size_t)cap * ((size_t)H + (size_t)HQ * K) + ((size_t)i * H + h) * V;
    }
};
__device__ __forceinline__ CaptureRow capture_row(float* capsule, int b, int cap, int H, int HQ, int K, int V) {
    return CaptureRow{capsule + (size_t)b * cap * ((size_t)H + (size_t)HQ * K + (size_t)H * V), cap, H, HQ, K, V};
}

__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x))); }

// Blocks are dispatched round-robin over the 8 XCDs of the chip (block i runs on XCD i % 8).  This
// maps the i-th block an XCD receives to a logical block so that groups of `gs` consecutive logical
// blocks (blocks that read the same q/k rows) stay on one XCD and share its L2, while consecutive
// groups go to different XCDs (which spreads one sequence's work over the whole chip).  Blocks past
// the last whole round of 8 * gs keep their index.
__device__ __forceinline__ int xcd_remap(int phys, int n, int gs) {
    const int round = 8 * gs;
    if (phys >= (n / round) * round) return phys;
    const int x = phys & 7, j = phys >> 3;
    return (8 * (j / gs) + x) * gs + (j % gs);
}

}  // namespace gdn
