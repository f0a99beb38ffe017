// kv_append.hip -- slot-mapped write of new tokens' K/V rows into the block
// pool, and the block-table gather used to check indexing.
//
// Append (ttlab page, section 4; drpranayjha page, "How PagedAttention pages
// the KV cache"): a request's KV grows one token row at a time inside its
// current physical block; the row of token i is slot % 16 of block slot / 16.
// The work is a scatter of rows of D * b bytes, so one thread moves 16 bytes:
// each row is read and written with fully coalesced 16-byte accesses.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

__global__ __launch_bounds__(256) void kv_append_kernel(
    const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    const int64_t* __restrict__ slot_mapping, int num_tokens, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, int num_blocks, int num_kv_heads, int row_bytes) {
    const int chunks_per_row = row_bytes / 16;
    const int64_t total = (int64_t)num_tokens * num_kv_heads * chunks_per_row;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(idx % chunks_per_row);
        const int64_t row = idx / chunks_per_row;  // token * H + g
        const int g = (int)(row % num_kv_heads);
        const int64_t tok = row / num_kv_heads;
        const int64_t slot = slot_mapping[tok];
        if (slot < 0 || slot >= (int64_t)num_blocks * kBlock) continue;
        const size_t dst = cache_row_offset(slot / kBlock, g, (int)(slot % kBlock), num_kv_heads,
                                            row_bytes) + (size_t)c * 16;
        const size_t src = (size_t)row * row_bytes + (size_t)c * 16;
        const uint4 kk = *reinterpret_cast<const uint4*>(k + src);
        const uint4 vv = *reinterpret_cast<const uint4*>(v + src);
        *reinterpret_cast<uint4*>(k_cache + dst) = kk;
        *reinterpret_cast<uint4*>(v_cache + dst) = vv;
    }
}

hipError_t launch_kv_append(const void* k, const void* v, int elem_bytes,
                            const int64_t* slot_mapping, int num_tokens, void* k_cache,
                            void* v_cache, int num_blocks, int num_kv_heads, int head_dim,
                            hipStream_t stream) {
    if (num_tokens == 0) return hipSuccess;
    const int row_bytes = head_dim * elem_bytes;
    const int64_t total = (int64_t)num_tokens * num_kv_heads * (row_bytes / 16);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v),
                       slot_mapping, num_tokens, static_cast<uint8_t*>(k_cache),
                       static_cast<uint8_t*>(v_cache), num_blocks, num_kv_heads, row_bytes);
    return hipGetLastError();
}

// Gather: out[s][g][t][:] = cache row of position t of sequence s through its
// block table, for t < min(n, max_ctx). A sequence with an out-of-range length
// or block id is skipped (checked per row before any cache access).
__global__ __launch_bounds__(256) void gather_kernel(
    const uint8_t* __restrict__ k_cache, const uint8_t* __restrict__ v_cache, int num_blocks,
    int num_kv_heads, int row_bytes, const int32_t* __restrict__ block_tables,
    int max_blocks_per_seq, const int32_t* __restrict__ context_lens, int num_seqs, int max_ctx,
    uint8_t* __restrict__ k_out, uint8_t* __restrict__ v_out) {
    const int chunks_per_row = row_bytes / 16;
    const int64_t total = (int64_t)num_seqs * num_kv_heads * max_ctx * chunks_per_row;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(idx % chunks_per_row);
        int64_t r = idx / chunks_per_row;
        const int t = (int)(r % max_ctx);
        r /= max_ctx;
        const int g = (int)(r % num_kv_heads);
        const int s = (int)(r / num_kv_heads);
        const int n = context_lens[s];
        if (t >= n || n > max_blocks_per_seq * kBlock) continue;
        const int64_t blk = block_tables[(int64_t)s * max_blocks_per_seq + t / kBlock];
        if (blk < 0 || blk >= num_blocks) continue;
        const size_t src = cache_row_offset(blk, g, t % kBlock, num_kv_heads, row_bytes) + c * 16;
        const size_t dst = (((size_t)s * num_kv_heads + g) * max_ctx + t) * row_bytes + c * 16;
        *reinterpret_cast<uint4*>(k_out + dst) = *reinterpret_cast<const uint4*>(k_cache + src);
        *reinterpret_cast<uint4*>(v_out + dst) = *reinterpret_cast<const uint4*>(v_cache + src);
    }
}

hipError_t launch_gather(const void* k_cache, const void* v_cache, int elem_bytes,
                         int num_blocks, int num_kv_heads, int head_dim,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_seqs, int max_ctx, void* k_out,
                         void* v_out, hipStream_t stream) {
    const int row_bytes = head_dim * elem_bytes;
    const int64_t total = (int64_t)num_seqs * num_kv_heads * max_ctx * (row_bytes / 16);
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(k_cache), static_cast<const uint8_t*>(v_cache),
                       num_blocks, num_kv_heads, row_bytes, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, max_ctx, static_cast<uint8_t*>(k_out),
                       static_cast<uint8_t*>(v_out));
    return hipGetLastError();
}

}  // namespace pkv
