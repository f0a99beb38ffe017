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

inline size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspaces keep float scratch at the front and the int32 counters (which
// must be zero when a call starts, and are left zero by every call) in the
// last bytes. Float scratch of any call fits below the counters of any other
// call sized no larger, so one workspace, zeroed once and sized for the
// largest shape, serves every smaller call without clearing it again.
//
// Decode: 2 * workers partial slots (balanced split) or one slot per
// (sequence, KV head, partition) (fixed partitions) at the front, counters
// [S][H_kv] at the end, each part a multiple of 256 bytes.
inline size_t decode_slot_bytes(int num_q_heads, int num_kv_heads, int head_dim, int workers) {
    const int gm = padded_group(num_q_heads / num_kv_heads);
    return round256((size_t)2 * workers * decode_slot_floats(gm, head_dim) * sizeof(float));
}
inline size_t decode_counter_bytes(int num_seqs, int num_kv_heads) {
    return round256((size_t)num_seqs * num_kv_heads * sizeof(int32_t));
}
// Fixed partitions of partition_size tokens: one slot per (sequence, KV head,
// partition), ceil(max_blocks_per_seq * 16 / partition_size) partitions.
inline int decode_partitions(int max_blocks_per_seq, int partition_size) {
    const int pt = partition_size / 16;
    return (max_blocks_per_seq + pt - 1) / pt;
}
inline size_t decode_partition_slot_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                          int head_dim, int max_blocks_per_seq,
                                          int partition_size) {
    const int gm = padded_group(num_q_heads / num_kv_heads);
    return round256((size_t)num_seqs * num_kv_heads *
                    decode_partitions(max_blocks_per_seq, partition_size) *
                    decode_slot_floats(gm, head_dim) * sizeof(float));
}
inline size_t decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                     int head_dim, int max_blocks_per_seq, int partition_size,
                                     int workers) {
    const size_t slots =
        partition_size > 0
            ? decode_partition_slot_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                          max_blocks_per_seq, partition_size)
            : decode_slot_bytes(num_q_heads, num_kv_heads, head_dim, workers);
    return slots + decode_counter_bytes(num_seqs, num_kv_heads);
}
// Start of the last `bytes` bytes of a workspace of ws_bytes (256-aligned).
inline size_t tail_offset(size_t ws_bytes, size_t bytes) { return (ws_bytes & ~(size_t)255) - bytes; }

// ---- shared-prefix decode ----------------------------------------------------
// The prefix pass runs workgroups of 128 (member, query head) rows of one
// prefix group and KV head over one chunk of the prefix blocks, and a
// prefill with few query rows splits each row tile's keys the same way; the
// chunk count aims at this many workgroups: one per CU of an MI355X. Eight
// 16-token chunks over 8192-token contexts (32 / 8 heads) take 52.8 us at
// 256 (four chunks per row tile), 56.3 at 512, 59-61 at 192, 320 and 384,
// and 65-79 at 128, 768 and 1024.
constexpr int kPrefixTargetWorkgroups = 256;
// Partial slots of 16 rows in the workspace. The chunk count is capped so
// that the slots of chunked groups fit; an unchunked group needs none.
constexpr int kPrefixSlots = 4096;

// One prefix partial: accumulators [16 rows][D], then 16 maxima and 16 sums.
constexpr int prefix_slot_floats(int d) { return 16 * d + 32; }

// Row blocks of 16 (member, head) rows over all groups, at most.
inline int64_t prefix_row_blocks_bound(int num_seqs, int group, int num_groups) {
    return ((int64_t)num_seqs * group + 15) / 16 + num_groups;
}
// Prefix workgroups, at most: H * (128-row tiles) with one chunk; with more
// chunks (ceil(target / (H * tiles)) of them) fewer than target + H * tiles.
inline int64_t prefix_workgroup_bound(int num_seqs, int group, int num_kv_heads, int num_groups) {
    const int64_t tiles = ((int64_t)num_seqs * group + 127) / 128 + num_groups;
    return (int64_t)num_kv_heads * tiles + kPrefixTargetWorkgroups;
}

// Byte offsets in the shared-prefix workspace. Front: the suffix pass's
// decode slots, the float32 suffix results [S][H_q][D] and [S][H_q], and
// kPrefixSlots prefix partial slots. End: the suffix pass's counters
// [S][H_kv].
struct SharedPrefixLayout {
    size_t res_o, res_lse, prefix_slots, floats;   // float part (from the start)
    size_t decode_counter_bytes;
    size_t total;
};
inline SharedPrefixLayout shared_prefix_layout(int num_seqs, int num_q_heads, int num_kv_heads,
                                               int head_dim, int workers) {
    SharedPrefixLayout l;
    size_t off = decode_slot_bytes(num_q_heads, num_kv_heads, head_dim, workers);
    l.res_o = off;
    off += round256((size_t)num_seqs * num_q_heads * head_dim * sizeof(float));
    l.res_lse = off;
    off += round256((size_t)num_seqs * num_q_heads * sizeof(float));
    l.prefix_slots = off;
    off += round256((size_t)kPrefixSlots * prefix_slot_floats(head_dim) * sizeof(float));
    l.floats = off;
    l.decode_counter_bytes = decode_counter_bytes(num_seqs, num_kv_heads);
    l.total = l.floats + l.decode_counter_bytes;
    return l;
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
    int partition_size = 0;  // tokens per fixed partition (a multiple of 16); 0 = balanced split
    int* counters;    // [S][H_kv], zero on entry
    float* slots;     // partial slots
    void* out;
    hipStream_t stream;
    // Shared-prefix decode only. With res_o set, the decode launch is the
    // suffix pass: grouped sequences skip their shared blocks and leave
    // float32 results in res_o / res_lse instead of writing out.
    int num_groups = 0;
    const int32_t* group_starts = nullptr;  // [num_groups + 1] (device)
    const int32_t* group_prefix = nullptr;  // [num_groups] (device)
    float* res_o = nullptr;                 // [S][H_q][D]
    float* res_lse = nullptr;               // [S][H_q]
    float* prefix_slots = nullptr;          // prefix pass: partial slots
};

// Paged chunked-prefill attention (paged_prefill.hip).
struct PrefillArgs {
    const void* q;
    int q_dtype;
    int kv_dtype;
    int num_seqs;
    int num_tokens;  // rows of q and out
    int num_q_heads;
    int num_kv_heads;
    int group;
    int head_dim;
    int num_blocks;
    const void* k_cache;
    const void* v_cache;
    const int32_t* query_start;  // [S + 1] (device)
    const int32_t* block_tables;
    int max_blocks_per_seq;
    const int32_t* context_lens;
    float scale;
    float k_scale;
    float v_scale;
    float* slots = nullptr;  // kPrefixSlots partial slots: few-row sequences split their keys
    void* out;
    hipStream_t stream;
};
hipError_t launch_paged_prefill(const PrefillArgs& a);
// Workgroups one prefill launch starts at most (its grid).
int64_t prefill_task_bound(int num_seqs, int num_tokens, int group, int num_kv_heads);

hipError_t launch_kv_append(const void* k, const void* v, int elem_bytes,
                            const int64_t* slot_mapping, int num_tokens, void* k_cache,
                            void* v_cache, int num_blocks, int num_kv_heads, int head_dim,
                            hipStream_t stream);

hipError_t launch_kv_append_fp8(const void* k, const void* v, int src_dtype,
                                const int64_t* slot_mapping, int num_tokens, void* k_cache,
                                void* v_cache, int num_blocks, int num_kv_heads, int head_dim,
                                float k_scale, float v_scale, hipStream_t stream);

hipError_t launch_paged_decode(const DecodeArgs& a);

// The streaming-read yardstick (stream_read.hip).
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int num_workgroups,
                              hipStream_t stream);

// The shared-prefix decode: the suffix pass (launch_paged_decode with res_o
// set), then the prefix pass that merges and writes out.
hipError_t launch_shared_prefix(const DecodeArgs& a);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, int elem_bytes, int num_blocks,
                              int num_kv_heads, int head_dim, const int32_t* pairs,
                              int num_pairs, hipStream_t stream);

hipError_t launch_gather(const void* k_cache, const void* v_cache, int elem_bytes,
                         int num_blocks, int num_kv_heads, int head_dim,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_seqs, int max_ctx, void* k_out,
                         void* v_out, hipStream_t stream);

}  // namespace pkv
