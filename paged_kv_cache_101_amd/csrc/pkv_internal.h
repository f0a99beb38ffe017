// pkv_internal.h -- host-side launchers behind the C ABI. Arguments reaching
// these functions have been validated by pkv_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

// Worker waves of one decode launch (the device default fills every CU).
constexpr int kMaxWorkers = PKV_MAX_WORKERS;

// Query heads per KV head are handled in register groups of 1, 2, 4, 6 or 8.
constexpr int padded_group(int g) { return g <= 1 ? 1 : g <= 2 ? 2 : g <= 4 ? 4 : g <= 6 ? 6 : 8; }

// One partial in the decode workspace: the unnormalised accumulator of GM
// heads x D, then GM maxima and GM sums, padded to a multiple of 4 floats.
constexpr int decode_slot_floats(int gm, int d) { return gm * d + ((2 * gm + 3) & ~3); }

// Decode workspace: int32 counters [S][H_kv] (rounded up to 256 bytes), then
// 2 * workers partial slots.
inline size_t decode_counter_bytes(int num_seqs, int num_kv_heads) {
    return (((size_t)num_seqs * num_kv_heads * sizeof(int32_t)) + 255) & ~(size_t)255;
}
inline size_t decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                     int head_dim, int workers) {
    const int gm = padded_group(num_q_heads / num_kv_heads);
    return decode_counter_bytes(num_seqs, num_kv_heads) +
           (size_t)2 * workers * decode_slot_floats(gm, head_dim) * sizeof(float);
}

struct DecodeArgs {
    const void* q;
    int q_dtype;
    int kv_dtype;
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int group;  // G = H_q / H_kv
    int head_dim;
    int num_blocks;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    int max_blocks_per_seq;
    const int32_t* context_lens;
    float scale;
    float k_scale;
    float v_scale;
    int num_workers;  // 0 = fill the device
    int* counters;    // [S][H_kv], zero on entry
    float* slots;     // partial slots
    void* out;
    hipStream_t stream;
};

hipError_t launch_kv_append(const void* k, const void* v, int elem_bytes,
                            const int64_t* slot_mapping, int num_tokens, void* k_cache,
                            void* v_cache, int num_blocks, int num_kv_heads, int head_dim,
                            hipStream_t stream);

hipError_t launch_kv_append_fp8(const void* k, const void* v, int src_dtype,
                                const int64_t* slot_mapping, int num_tokens, void* k_cache,
                                void* v_cache, int num_blocks, int num_kv_heads, int head_dim,
                                float k_scale, float v_scale, hipStream_t stream);

hipError_t launch_paged_decode(const DecodeArgs& a);

hipError_t launch_gather(const void* k_cache, const void* v_cache, int elem_bytes,
                         int num_blocks, int num_kv_heads, int head_dim,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_seqs, int max_ctx, void* k_out,
                         void* v_out, hipStream_t stream);

}  // namespace pkv
