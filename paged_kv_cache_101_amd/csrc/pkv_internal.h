// pkv_internal.h -- host-side launchers behind the C ABI. Arguments reaching
// these functions have been validated by pkv_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

// Tokens of one partition are scored into LDS, so a partition is bounded.
constexpr int kMaxPartition = PKV_MAX_PARTITION;

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
    int partition_size;
    int num_partitions;
    float* ws_m;  // [S][H_q][Pn] (natural-log units), only when Pn > 1
    float* ws_l;  // [S][H_q][Pn]
    float* ws_o;  // [S][H_q][Pn][D]
    void* out;
    hipStream_t stream;
};

hipError_t launch_kv_append(const void* k, const void* v, int elem_bytes,
                            const int64_t* slot_mapping, int num_tokens, void* k_cache,
                            void* v_cache, int num_blocks, int num_kv_heads, int head_dim,
                            hipStream_t stream);

hipError_t launch_paged_decode(const DecodeArgs& a);

hipError_t launch_gather(const void* k_cache, const void* v_cache, int elem_bytes,
                         int num_blocks, int num_kv_heads, int head_dim,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_seqs, int max_ctx, void* k_out,
                         void* v_out, hipStream_t stream);

}  // namespace pkv
