// pkv_device.h -- device-side building blocks shared by the libpkv kernels:
// element types, the cache addressing, cross-lane reductions (DPP within a
// 16-lane row, swizzles across rows) and round-to-nearest-even stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kBlock = PKV_BLOCK_SIZE;  // tokens per physical block
constexpr int kWave = 64;               // CDNA wavefront width
constexpr int kElemsPerLane = 8;        // cache elements a lane owns per row chunk

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

template <int DT>
struct Elem;
template <>
struct Elem<PKV_F32> {
    static constexpr int bytes = 4;
};
template <>
struct Elem<PKV_F16> {
    static constexpr int bytes = 2;
};
template <>
struct Elem<PKV_BF16> {
    static constexpr int bytes = 2;
};
template <>
struct Elem<PKV_FP8_E4M3> {
    static constexpr int bytes = 1;
};

// Byte offset of row `off` of tile (blk, g) in a [num_blocks][H][16][D] cache
// with `row_bytes` = D * element bytes. The only place the layout is spelled
// out on the device: decode, gather and append all go through it.
__device__ __forceinline__ size_t cache_row_offset(int64_t blk, int g, int off, int num_kv_heads,
                                                   int row_bytes) {
    return ((size_t)(blk * num_kv_heads + g) * kBlock + off) * (size_t)row_bytes;
}

// 8 elements held by one lane, as raw dwords (f32: 8, 16-bit: 4, fp8: 2).
template <int DT>
struct Chunk {
    static constexpr int dwords = Elem<DT>::bytes * kElemsPerLane / 4;
    uint32_t w[dwords];
};

// Loads of 8 elements through a plain pointer (optionally nontemporal).
template <typename V>
__device__ __forceinline__ V load_vec(const uint8_t* p, bool stream) {
    const V* q = reinterpret_cast<const V*>(p);
    return stream ? __builtin_nontemporal_load(q) : *q;
}

template <int DT, bool STREAM = false>
__device__ __forceinline__ Chunk<DT> load_chunk(const uint8_t* p) {
    Chunk<DT> c;
    if constexpr (Chunk<DT>::dwords == 8) {
        u32x4_t a = load_vec<u32x4_t>(p, STREAM);
        u32x4_t b = load_vec<u32x4_t>(p + 16, STREAM);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c.w[i] = a[i];
            c.w[4 + i] = b[i];
        }
    } else if constexpr (Chunk<DT>::dwords == 4) {
        u32x4_t a = load_vec<u32x4_t>(p, STREAM);
#pragma unroll
        for (int i = 0; i < 4; ++i) c.w[i] = a[i];
    } else {
        u32x2_t a = load_vec<u32x2_t>(p, STREAM);
        c.w[0] = a[0];
        c.w[1] = a[1];
    }
    return c;
}

// Buffer resource for `bytes` bytes at `base` (raw, untyped dwords). Loads
// through it outside [0, bytes) return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// 8 elements at byte `voff` of a buffer, nontemporal (streamed past the
// caches). The address lives in one 32-bit VGPR plus the scalar resource.
template <int DT>
__device__ __forceinline__ Chunk<DT> load_chunk_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    constexpr int kNontemporal = 2;
    Chunk<DT> c;
    if constexpr (Chunk<DT>::dwords == 8) {
        u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kNontemporal);
        u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, 0, kNontemporal);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c.w[i] = a[i];
            c.w[4 + i] = b[i];
        }
    } else if constexpr (Chunk<DT>::dwords == 4) {
        u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kNontemporal);
#pragma unroll
        for (int i = 0; i < 4; ++i) c.w[i] = a[i];
    } else {
        u32x2_t a = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, kNontemporal);
        c.w[0] = a[0];
        c.w[1] = a[1];
    }
    return c;
}

template <int DT>
__device__ __forceinline__ void zero_chunk(Chunk<DT>& c) {
#pragma unroll
    for (int i = 0; i < Chunk<DT>::dwords; ++i) c.w[i] = 0u;
}

// The 8 elements of a chunk as float32 (exact for every storage type).
// fp8: the hardware OCP E4M3FN -> f32 conversion, two bytes per instruction.
template <int DT>
__device__ __forceinline__ void chunk_to_f32(const Chunk<DT>& c, float* f) {
    if constexpr (DT == PKV_F32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = __builtin_bit_cast(float, c.w[i]);
    } else if constexpr (DT == PKV_F16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            half2_t h = __builtin_bit_cast(half2_t, c.w[i]);
            f[2 * i] = (float)h.x;
            f[2 * i + 1] = (float)h.y;
        }
    } else if constexpr (DT == PKV_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __builtin_bit_cast(float, c.w[i] << 16);
            f[2 * i + 1] = __builtin_bit_cast(float, c.w[i] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(c.w[i], false);
            auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(c.w[i], true);
            f[4 * i] = lo[0];
            f[4 * i + 1] = lo[1];
            f[4 * i + 2] = hi[0];
            f[4 * i + 3] = hi[1];
        }
    }
}

// float32 -> storage type with round-to-nearest-even (the default rounding
// mode for the f16 conversion; bf16 by the carry-propagating add on the bit
// pattern, NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <int DT>
__device__ __forceinline__ void store_f32_as(void* base, size_t idx, float x) {
    if constexpr (DT == PKV_F32) {
        reinterpret_cast<float*>(base)[idx] = x;
    } else if constexpr (DT == PKV_F16) {
        reinterpret_cast<_Float16*>(base)[idx] = (_Float16)x;
    } else {
        static_assert(DT == PKV_BF16, "output type");
        reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16_rne(x);
    }
}

// ---- cross-lane reductions -------------------------------------------------

// DPP controls (CDNA): quad permutations, mirrors inside a 16-lane row.
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N = 4, 8 or 16, all inside one row);
// every lane of the group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N == 4 || N == 8 || N == 16, "group size");
    v += dpp<kDppQuadXor1>(v);
    v += dpp<kDppQuadXor2>(v);
    if constexpr (N >= 8) v += dpp<kDppRowHalfMirror>(v);
    if constexpr (N >= 16) v += dpp<kDppRowMirror>(v);
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
    v = group_sum<16>(v);
    v += __shfl_xor(v, 16, kWave);
    v += __shfl_xor(v, 32, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<kDppQuadXor1>(v));
    v = fmaxf(v, dpp<kDppQuadXor2>(v));
    v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
    v = fmaxf(v, dpp<kDppRowMirror>(v));
    v = fmaxf(v, __shfl_xor(v, 16, kWave));
    v = fmaxf(v, __shfl_xor(v, 32, kWave));
    return v;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Wave index as a scalar (wave-uniform) value.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

}  // namespace pkv
