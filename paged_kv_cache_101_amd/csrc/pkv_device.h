// pkv_device.h -- device-side building blocks shared by the libpkv kernels:
// element types, the in-block cache layout, cross-lane reductions (DPP within
// a 16-lane row, swizzles across rows) and round-to-nearest-even stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kBlock = PKV_BLOCK_SIZE;  // tokens per physical block
constexpr int kWave = 64;               // CDNA wavefront width

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

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

// Cache layout. The pool is [num_blocks][H][16 * D] elements: one tile of 16
// tokens x D elements per (physical block, KV head), tiles contiguous. Inside a
// tile the two caches are ordered for the matrix-core operands of decode:
//   K: [D/8][16][8]  token t, element e at ((e / 8) * 16 + t) * 8 + e % 8
//      (8-element slabs: the 16 tokens' slab i lie together, so the slabs a
//      QK instruction consumes are one contiguous run);
//   V: token t, element e = 16 * j + c (element column c of 16-element block
//      j) at (((j / 2) * 16 + c) * 4 + t / 4) * 8 + (j % 2) * 4 + t % 4
//      (P.V contracts over tokens: 4 consecutive tokens of one element
//      column, for two neighbouring element blocks, form one 8-element run,
//      and the 64 runs of a block pair are contiguous).
// These three functions are the only place the layout is spelled out on the
// device: decode, gather and append all go through them.
__device__ __forceinline__ size_t tile_elem_offset(int64_t blk, int g, int num_kv_heads, int d) {
    return (size_t)(blk * num_kv_heads + g) * kBlock * (size_t)d;
}
__device__ __forceinline__ int k_elem_index(int t, int e) {
    return ((e >> 3) * kBlock + t) * 8 + (e & 7);
}
__device__ __forceinline__ int v_elem_index(int t, int e) {
    const int j = e >> 4, c = e & 15;
    return ((((j >> 1) * kBlock + c) * 4 + (t >> 2)) * 2 + (j & 1)) * 4 + (t & 3);
}

// Buffer resource for `bytes` bytes at `base` (raw, untyped dwords). Loads
// through it outside [0, bytes) return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
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

// The four 16-lane rows' results (every lane of a row holding its row's),
// combined into one wave-uniform value: lanes 0, 16, 32 and 48 are read into
// scalar registers rather than exchanged through the LDS crossbar.
template <typename Op>
__device__ __forceinline__ float combine_rows(float v, Op op) {
    auto rd = [&](int l) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
    };
    return op(op(rd(0), rd(16)), op(rd(32), rd(48)));
}

__device__ __forceinline__ float wave_sum(float v) {
    return combine_rows(group_sum<16>(v), [](float x, float y) { return x + y; });
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<kDppQuadXor1>(v));
    v = fmaxf(v, dpp<kDppQuadXor2>(v));
    v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
    v = fmaxf(v, dpp<kDppRowMirror>(v));
    return combine_rows(v, [](float x, float y) { return fmaxf(x, y); });
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Wave index as a scalar (wave-uniform) value.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

}  // namespace pkv
