// kv_append.hip -- slot-mapped write of new tokens' K/V rows into the block
// pool, and the block-table gather used to check indexing.
//
// Append (ttlab page, section 4; drpranayjha page, "How PagedAttention pages
// the KV cache"): a request's KV grows one token row at a time inside its
// current physical block; the row of token i is slot % 16 of block slot / 16.
// One thread moves one 8-element group of a (token, KV head) row: the K group
// is one contiguous slab entry of the tile, the V group eight elements, one in
// each of eight element rows of the tile (the in-block layout is in
// pkv_device.h).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

// 8 elements of `eb` bytes: one 32-, 16- or 8-byte copy.
__device__ __forceinline__ void copy8(uint8_t* dst, const uint8_t* src, int eb) {
    if (eb == 4) {
        reinterpret_cast<uint4*>(dst)[0] = reinterpret_cast<const uint4*>(src)[0];
        reinterpret_cast<uint4*>(dst)[1] = reinterpret_cast<const uint4*>(src)[1];
    } else if (eb == 2) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    } else {
        *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
    }
}

// One element of `eb` bytes.
__device__ __forceinline__ void copy1(uint8_t* dst, const uint8_t* src, int eb) {
    if (eb == 4)
        *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(src);
    else if (eb == 2)
        *reinterpret_cast<uint16_t*>(dst) = *reinterpret_cast<const uint16_t*>(src);
    else
        *dst = *src;
}

}  // namespace

// One 8-element group of EB-byte elements as dwords (EB 1: 2, 2: 4, 4: 8).
template <int EB>
struct Group {
    uint32_t w[2 * EB];
    __device__ __forceinline__ void load(const uint8_t* src) {
        if constexpr (EB == 1) {
            const uint2 a = *reinterpret_cast<const uint2*>(src);
            w[0] = a.x, w[1] = a.y;
        } else {
#pragma unroll
            for (int i = 0; i < EB / 2; ++i) {
                const uint4 a = reinterpret_cast<const uint4*>(src)[i];
                w[4 * i] = a.x, w[4 * i + 1] = a.y, w[4 * i + 2] = a.z, w[4 * i + 3] = a.w;
            }
        }
    }
    __device__ __forceinline__ void store(uint8_t* dst) const {
        if constexpr (EB == 1) {
            *reinterpret_cast<uint2*>(dst) = uint2{w[0], w[1]};
        } else {
#pragma unroll
            for (int i = 0; i < EB / 2; ++i)
                reinterpret_cast<uint4*>(dst)[i] = uint4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
        }
    }
    // element e (0..7)
    __device__ __forceinline__ void store_elem(uint8_t* dst, int e) const {
        if constexpr (EB == 4)
            *reinterpret_cast<uint32_t*>(dst) = w[e];
        else if constexpr (EB == 2)
            *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        else
            *dst = (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
    }
};

template <int EB>
__global__ __launch_bounds__(256) void kv_append_kernel(
    const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    const int64_t* __restrict__ slot_mapping, int num_tokens, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, int num_blocks, int num_kv_heads, int head_dim) {
    const int groups = head_dim / 8;
    const int64_t total = (int64_t)num_tokens * num_kv_heads * groups;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(idx % groups);
        const int64_t row = idx / groups;  // token * H + g
        const int g = (int)(row % num_kv_heads);
        const int64_t tok = row / num_kv_heads;
        // The source group's address does not depend on the slot, so its K
        // and V are read together with the slot: one memory latency, not two.
        const size_t src = ((size_t)row * head_dim + (size_t)c * 8) * EB;
        Group<EB> kg, vg;
        kg.load(k + src);
        vg.load(v + src);
        const int64_t slot = slot_mapping[tok];
        if (slot < 0 || slot >= (int64_t)num_blocks * kBlock) continue;
        const int t = (int)(slot % kBlock);
        const size_t tile = tile_elem_offset(slot / kBlock, g, num_kv_heads, head_dim);
        kg.store(k_cache + (tile + k_elem_index(t, c * 8)) * EB);
#pragma unroll
        for (int e = 0; e < 8; ++e) vg.store_elem(v_cache + (tile + v_elem_index(t, c * 8 + e)) * EB, e);
    }
}

// ---- quantising append into an fp8 cache -------------------------------------
//
// (ttlab page, section 2: fp8 storage halves the bytes per element again.)
// Each element x of a float32 / float16 / bfloat16 row is stored as the OCP
// E4M3FN code of y = x / scale, the quotient taken in float32 (IEEE, round to
// nearest even), with k_scale for K and v_scale for V.

// E4M3FN code of a float32 value, from the format's definition (sign, 4
// exponent bits with bias 7, 3 mantissa bits, no infinity, 0x7F / 0xFF NaN,
// largest finite 448): round to nearest, ties to the even mantissa; values
// beyond +-448 (and infinities) saturate to +-448; NaN becomes 0x7F.
__device__ __forceinline__ uint32_t fp8_e4m3_code(float y) {
    if (y != y) return 0x7Fu;
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fabsf(y);
    if (a >= 448.f) return sign | 0x7Eu;
    if (a < 0.015625f)  // below 2^-6: multiples of 2^-9 (8 * 2^-9 is the smallest normal)
        return sign | (uint32_t)__builtin_rintf(a * 512.f);
    // normal: keep 3 of float32's 23 mantissa bits with round to nearest even
    // (a carry moves the exponent), then rebias the exponent from 127 to 7
    const uint32_t b = __float_as_uint(a);
    return sign | (((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - (120u << 3));
}

template <int SRC>
__device__ __forceinline__ void load8_f32(const uint8_t* p, float* f) {
    if constexpr (SRC == PKV_F32) {
        const float4 a = reinterpret_cast<const float4*>(p)[0];
        const float4 b = reinterpret_cast<const float4*>(p)[1];
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    } else {
        const uint4 a = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (SRC == PKV_F16) {
                f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
                f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
            } else {
                f[2 * i] = __uint_as_float(w[i] << 16);
                f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
            }
        }
    }
}

template <int SRC>
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(
    const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    const int64_t* __restrict__ slot_mapping, int num_tokens, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, int num_blocks, int num_kv_heads, int head_dim, float k_scale,
    float v_scale) {
    constexpr int SB = Elem<SRC>::bytes;
    const int groups = head_dim / 8;
    const int64_t total = (int64_t)num_tokens * num_kv_heads * groups;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(idx % groups);
        const int64_t row = idx / groups;  // token * H + g
        const int g = (int)(row % num_kv_heads);
        const int64_t tok = row / num_kv_heads;
        // the source rows are read together with the slot (their addresses
        // do not depend on it)
        const size_t src = ((size_t)row * head_dim + (size_t)c * 8) * SB;
        float kf[8], vf[8];
        load8_f32<SRC>(k + src, kf);
        load8_f32<SRC>(v + src, vf);
        const int64_t slot = slot_mapping[tok];
        if (slot < 0 || slot >= (int64_t)num_blocks * kBlock) continue;
        const int t = (int)(slot % kBlock);
        const size_t tile = tile_elem_offset(slot / kBlock, g, num_kv_heads, head_dim);
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            lo |= fp8_e4m3_code(kf[e] / k_scale) << (8 * e);
            hi |= fp8_e4m3_code(kf[4 + e] / k_scale) << (8 * e);
        }
        *reinterpret_cast<uint2*>(k_cache + tile + k_elem_index(t, c * 8)) = make_uint2(lo, hi);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            v_cache[tile + v_elem_index(t, c * 8 + e)] = (uint8_t)fp8_e4m3_code(vf[e] / v_scale);
    }
}

hipError_t launch_kv_append_fp8(const void* k, const void* v, int src_dtype,
                                const int64_t* slot_mapping, int num_tokens, void* k_cache,
                                void* v_cache, int num_blocks, int num_kv_heads, int head_dim,
                                float k_scale, float v_scale, hipStream_t stream) {
    if (num_tokens == 0) return hipSuccess;
    const int64_t total = (int64_t)num_tokens * num_kv_heads * (head_dim / 8);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    auto args = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v),
                           slot_mapping, num_tokens, static_cast<uint8_t*>(k_cache),
                           static_cast<uint8_t*>(v_cache), num_blocks, num_kv_heads, head_dim,
                           k_scale, v_scale);
    };
    if (src_dtype == PKV_F32)
        args(kv_append_fp8_kernel<PKV_F32>);
    else if (src_dtype == PKV_F16)
        args(kv_append_fp8_kernel<PKV_F16>);
    else
        args(kv_append_fp8_kernel<PKV_BF16>);
    return hipGetLastError();
}

hipError_t launch_kv_append(const void* k, const void* v, int elem_bytes,
                            const int64_t* slot_mapping, int num_tokens, void* k_cache,
                            void* v_cache, int num_blocks, int num_kv_heads, int head_dim,
                            hipStream_t stream) {
    if (num_tokens == 0) return hipSuccess;
    const int64_t total = (int64_t)num_tokens * num_kv_heads * (head_dim / 8);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    auto args = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v),
                           slot_mapping, num_tokens, static_cast<uint8_t*>(k_cache),
                           static_cast<uint8_t*>(v_cache), num_blocks, num_kv_heads, head_dim);
    };
    if (elem_bytes == 4)
        args(kv_append_kernel<4>);
    else if (elem_bytes == 2)
        args(kv_append_kernel<2>);
    else
        args(kv_append_kernel<1>);
    return hipGetLastError();
}

// Gather: out[s][g][t][:] = the K/V row of position t of sequence s through
// its block table, for t < min(n, max_ctx), in plain row order. A sequence with
// an out-of-range length or block id is skipped (checked per row before any
// cache access).
__global__ __launch_bounds__(256) void gather_kernel(
    const uint8_t* __restrict__ k_cache, const uint8_t* __restrict__ v_cache, int num_blocks,
    int num_kv_heads, int head_dim, int eb, const int32_t* __restrict__ block_tables,
    int max_blocks_per_seq, const int32_t* __restrict__ context_lens, int num_seqs, int max_ctx,
    uint8_t* __restrict__ k_out, uint8_t* __restrict__ v_out) {
    const int groups = head_dim / 8;
    const int64_t total = (int64_t)num_seqs * num_kv_heads * max_ctx * groups;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(idx % groups);
        int64_t r = idx / groups;
        const int t = (int)(r % max_ctx);
        r /= max_ctx;
        const int g = (int)(r % num_kv_heads);
        const int s = (int)(r / num_kv_heads);
        const int n = context_lens[s];
        if (t >= n || n > max_blocks_per_seq * kBlock) continue;
        const int64_t blk = block_tables[(int64_t)s * max_blocks_per_seq + t / kBlock];
        if (blk < 0 || blk >= num_blocks) continue;
        const size_t tile = tile_elem_offset(blk, g, num_kv_heads, head_dim);
        const int tb = t % kBlock;
        const size_t dst =
            ((((size_t)s * num_kv_heads + g) * max_ctx + t) * head_dim + (size_t)c * 8) * eb;
        copy8(k_out + dst, k_cache + (tile + k_elem_index(tb, c * 8)) * eb, eb);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            copy1(v_out + dst + (size_t)e * eb, v_cache + (tile + v_elem_index(tb, c * 8 + e)) * eb,
                  eb);
    }
}

// ---- whole-block copies (copy-on-write) ---------------------------------------
//
// (ttlab page, section 4: a block shared by several requests is copied before
// one of them writes into it.) A physical block's KV heads are contiguous in
// the pool -- (blk * H + g) tiles -- so a block is one run of H * 16 * D
// elements in each cache, copied 16 bytes per thread, the same bytes in the
// same in-tile order.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* __restrict__ k_cache,
                                                          uint8_t* __restrict__ v_cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int num_pairs, int num_blocks,
                                                          int64_t block_bytes) {
    const int64_t chunks = block_bytes / 16;  // 16-byte pieces of one block
    const int64_t total = (int64_t)num_pairs * chunks;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t pr = idx / chunks, c = idx % chunks;
        const int src = pairs[2 * pr], dst = pairs[2 * pr + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) continue;
        const int64_t s = (int64_t)src * block_bytes + c * 16, d = (int64_t)dst * block_bytes + c * 16;
        *reinterpret_cast<uint4*>(k_cache + d) = *reinterpret_cast<const uint4*>(k_cache + s);
        *reinterpret_cast<uint4*>(v_cache + d) = *reinterpret_cast<const uint4*>(v_cache + s);
    }
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, int elem_bytes, int num_blocks,
                              int num_kv_heads, int head_dim, const int32_t* pairs,
                              int num_pairs, hipStream_t stream) {
    if (num_pairs == 0) return hipSuccess;
    const int64_t block_bytes = (int64_t)num_kv_heads * kBlock * head_dim * elem_bytes;
    const int64_t total = (int64_t)num_pairs * (block_bytes / 16);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), pairs,
                       num_pairs, num_blocks, block_bytes);
    return hipGetLastError();
}

hipError_t launch_gather(const void* k_cache, const void* v_cache, int elem_bytes,
                         int num_blocks, int num_kv_heads, int head_dim,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_seqs, int max_ctx, void* k_out,
                         void* v_out, hipStream_t stream) {
    const int64_t total = (int64_t)num_seqs * num_kv_heads * max_ctx * (head_dim / 8);
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(k_cache), static_cast<const uint8_t*>(v_cache),
                       num_blocks, num_kv_heads, head_dim, elem_bytes, block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, max_ctx,
                       static_cast<uint8_t*>(k_out), static_cast<uint8_t*>(v_out));
    return hipGetLastError();
}

}  // namespace pkv
