// pkv_api.hip -- the extern "C" entry points of libpkv.so (declared and
// documented in include/pkv.h). Every argument the host can check is checked
// here, before any HIP call; the launchers in the kernel files only see
// validated arguments.
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "pkv.h"
#include "pkv_internal.h"

#define PKV_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

int elem_bytes(int dtype) {
    switch (dtype) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    default: return 0;
    }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Common checks of a cache descriptor.
int check_cache(const pkv_cache_desc* c) {
    if (c == nullptr) return PKV_ERR_INVALID_ARG;
    if (c->num_blocks <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0) return PKV_ERR_INVALID_ARG;
    if (c->block_size != PKV_BLOCK_SIZE) return PKV_ERR_UNSUPPORTED;
    if (c->head_dim != 64 && c->head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (elem_bytes(c->dtype) == 0) return PKV_ERR_UNSUPPORTED;
    if (c->dtype == PKV_FP8_E4M3 && !(c->k_scale > 0.f && c->v_scale > 0.f))
        return PKV_ERR_INVALID_ARG;
    return PKV_OK;
}

}  // namespace

PKV_EXPORT const char* pkv_status_string(int status) {
    switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP launch error";
    case PKV_ERR_TOO_LARGE:
        return "batch needs more scratch than the allocation-free entry point's static buffer";
    default: return "unknown status";
    }
}

PKV_EXPORT size_t pkv_kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t dtype) {
    const int b = elem_bytes(dtype);
    if (num_layers <= 0 || num_kv_heads <= 0 || head_dim <= 0 || b == 0) return 0;
    return (size_t)2 * num_layers * num_kv_heads * head_dim * b;
}

PKV_EXPORT size_t pkv_cache_tensor_bytes(const pkv_cache_desc* cache) {
    if (check_cache(cache) != PKV_OK) return 0;
    return (size_t)cache->num_blocks * cache->num_kv_heads * PKV_BLOCK_SIZE * cache->head_dim *
           elem_bytes(cache->dtype);
}

PKV_EXPORT int pkv_kv_append(const void* k, const void* v, int32_t kv_dtype,
                             const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
                             void* v_cache, const pkv_cache_desc* cache, hipStream_t stream) {
    int rc = check_cache(cache);
    if (rc != PKV_OK) return rc;
    if (num_tokens < 0) return PKV_ERR_INVALID_ARG;
    // a byte copy, or quantising float32 / float16 / bfloat16 rows into an fp8 cache
    const bool quantise = cache->dtype == PKV_FP8_E4M3 &&
                          (kv_dtype == PKV_F32 || kv_dtype == PKV_F16 || kv_dtype == PKV_BF16);
    if (kv_dtype != cache->dtype && !quantise) return PKV_ERR_UNSUPPORTED;
    if (k_cache == nullptr || v_cache == nullptr) return PKV_ERR_INVALID_ARG;
    if (num_tokens > 0 && (k == nullptr || v == nullptr || slot_mapping == nullptr))
        return PKV_ERR_INVALID_ARG;
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
        return PKV_ERR_INVALID_ARG;
    if (num_tokens == 0) return PKV_OK;
    hipError_t err =
        quantise ? pkv::launch_kv_append_fp8(k, v, kv_dtype, slot_mapping, num_tokens, k_cache,
                                             v_cache, cache->num_blocks, cache->num_kv_heads,
                                             cache->head_dim, cache->k_scale, cache->v_scale,
                                             stream)
                 : pkv::launch_kv_append(k, v, elem_bytes(cache->dtype), slot_mapping, num_tokens,
                                         k_cache, v_cache, cache->num_blocks, cache->num_kv_heads,
                                         cache->head_dim, stream);
    return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

namespace {

// The decode shape checks of the workspace-size functions.
bool decode_shape_ok(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t num_workers) {
    return num_seqs > 0 && num_q_heads > 0 && num_kv_heads > 0 && head_dim > 0 &&
           num_q_heads % num_kv_heads == 0 && num_q_heads / num_kv_heads <= 8 &&
           num_workers >= 0 && num_workers <= pkv::kMaxWorkers;
}

bool partition_ok(int32_t partition_size) {
    return partition_size >= 0 && partition_size % PKV_BLOCK_SIZE == 0;
}

}  // namespace

PKV_EXPORT size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t max_blocks_per_seq, int32_t partition_size,
                                             int32_t num_workers) {
    if (!decode_shape_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, num_workers) ||
        max_blocks_per_seq <= 0 || !partition_ok(partition_size))
        return 0;
    return pkv::decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                       max_blocks_per_seq, partition_size,
                                       num_workers == 0 ? pkv::kMaxWorkers : num_workers);
}

namespace {

// Checks shared by the attention entry points (all but the workspace size),
// filling the decode launch arguments. with_workspace: the call takes one.
int decode_args(pkv::DecodeArgs& a, const void* q, int32_t q_dtype, int32_t num_seqs,
                int32_t num_q_heads, const void* k_cache, const void* v_cache,
                const pkv_cache_desc* cache, const int32_t* block_tables,
                int32_t max_blocks_per_seq, const int32_t* context_lens, float scale,
                int32_t num_workers, bool with_workspace, void* workspace, void* out,
                hipStream_t stream) {
    int rc = check_cache(cache);
    if (rc != PKV_OK) return rc;
    if (num_seqs <= 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0)
        return PKV_ERR_INVALID_ARG;
    if ((int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE > INT32_MAX) return PKV_ERR_UNSUPPORTED;
    if (num_q_heads % cache->num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
    const int group = num_q_heads / cache->num_kv_heads;
    if (group > 8) return PKV_ERR_UNSUPPORTED;
    const int kv = cache->dtype;
    const bool pair_ok = (kv == PKV_F32 && q_dtype == PKV_F32) ||
                         (kv == PKV_F16 && q_dtype == PKV_F16) ||
                         (kv == PKV_BF16 && q_dtype == PKV_BF16) ||
                         (kv == PKV_FP8_E4M3 && (q_dtype == PKV_F16 || q_dtype == PKV_BF16));
    if (!pair_ok) return PKV_ERR_UNSUPPORTED;
    if (q == nullptr || k_cache == nullptr || v_cache == nullptr || block_tables == nullptr ||
        context_lens == nullptr || out == nullptr)
        return PKV_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return PKV_ERR_INVALID_ARG;
    if (!(scale == scale)) return PKV_ERR_INVALID_ARG;
    if (num_workers < 0) return PKV_ERR_INVALID_ARG;
    if (num_workers > pkv::kMaxWorkers) return PKV_ERR_UNSUPPORTED;
    if (with_workspace && (workspace == nullptr || ((uintptr_t)workspace & 255u) != 0))
        return PKV_ERR_WORKSPACE;

    a = pkv::DecodeArgs{};
    a.q = q;
    a.q_dtype = q_dtype;
    a.kv_dtype = kv;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = cache->num_kv_heads;
    a.group = group;
    a.head_dim = cache->head_dim;
    a.num_blocks = cache->num_blocks;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.scale = scale;
    a.k_scale = cache->k_scale;
    a.v_scale = cache->v_scale;
    a.num_workers = num_workers;
    a.slots = static_cast<float*>(workspace);  // counters: set by the entry point
    a.out = out;
    a.stream = stream;
    return PKV_OK;
}

}  // namespace

PKV_EXPORT int pkv_paged_attention_decode(const void* q, int32_t q_dtype, int32_t num_seqs,
                                          int32_t num_q_heads, const void* k_cache,
                                          const void* v_cache, const pkv_cache_desc* cache,
                                          const int32_t* block_tables,
                                          int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, float scale,
                                          int32_t partition_size, int32_t num_workers,
                                          void* workspace, size_t workspace_bytes, void* out,
                                          hipStream_t stream) {
    pkv::DecodeArgs a;
    const int rc = decode_args(a, q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache,
                               block_tables, max_blocks_per_seq, context_lens, scale, num_workers,
                               true, workspace, out, stream);
    if (rc != PKV_OK) return rc;
    if (!partition_ok(partition_size)) return PKV_ERR_INVALID_ARG;
    a.partition_size = partition_size;
    if (workspace_bytes < pkv_decode_workspace_bytes(num_seqs, num_q_heads, cache->num_kv_heads,
                                                     cache->head_dim, max_blocks_per_seq,
                                                     partition_size, num_workers))
        return PKV_ERR_WORKSPACE;
    a.counters = reinterpret_cast<int*>(
        static_cast<char*>(workspace) +
        pkv::tail_offset(workspace_bytes, pkv::decode_counter_bytes(num_seqs, cache->num_kv_heads)));
    hipError_t err = pkv::launch_paged_decode(a);
    return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

PKV_EXPORT size_t pkv_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                    int32_t num_kv_heads, int32_t head_dim,
                                                    int32_t num_groups, int32_t num_workers) {
    if (!decode_shape_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, num_workers) ||
        num_groups < 0 || num_groups > num_seqs)
        return 0;
    return pkv::shared_prefix_layout(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                     num_workers == 0 ? pkv::kMaxWorkers : num_workers)
        .total;
}

PKV_EXPORT int pkv_paged_attention_decode_shared_prefix(
    const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads, const void* k_cache,
    const void* v_cache, const pkv_cache_desc* cache, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_groups,
    const int32_t* group_starts, const int32_t* group_prefix_blocks, float scale,
    int32_t num_workers, void* workspace, size_t workspace_bytes, void* out, hipStream_t stream) {
    pkv::DecodeArgs a;
    const int rc = decode_args(a, q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache,
                               block_tables, max_blocks_per_seq, context_lens, scale, num_workers,
                               true, workspace, out, stream);
    if (rc != PKV_OK) return rc;
    if (num_groups < 0 || num_groups > num_seqs) return PKV_ERR_INVALID_ARG;
    if (num_groups > 0 && (group_starts == nullptr || group_prefix_blocks == nullptr))
        return PKV_ERR_INVALID_ARG;
    if (workspace_bytes < pkv_shared_prefix_workspace_bytes(num_seqs, num_q_heads,
                                                            cache->num_kv_heads, cache->head_dim,
                                                            num_groups, num_workers))
        return PKV_ERR_WORKSPACE;
    const pkv::SharedPrefixLayout l =
        pkv::shared_prefix_layout(num_seqs, num_q_heads, cache->num_kv_heads, cache->head_dim,
                                  num_workers == 0 ? pkv::kMaxWorkers : num_workers);
    char* ws = static_cast<char*>(workspace);
    const size_t dctr = pkv::tail_offset(workspace_bytes, l.decode_counter_bytes);
    a.counters = reinterpret_cast<int*>(ws + dctr);
    hipError_t err;
    if (num_groups == 0) {
        err = pkv::launch_paged_decode(a);  // no prefix groups: plain decode
    } else {
        a.num_groups = num_groups;
        a.group_starts = group_starts;
        a.group_prefix = group_prefix_blocks;
        a.res_o = reinterpret_cast<float*>(ws + l.res_o);
        a.res_lse = reinterpret_cast<float*>(ws + l.res_lse);
        a.prefix_slots = reinterpret_cast<float*>(ws + l.prefix_slots);
        err = pkv::launch_shared_prefix(a);
    }
    return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

PKV_EXPORT size_t pkv_prefill_workspace_bytes(int32_t head_dim) {
    if (head_dim != 64 && head_dim != 128) return 0;
    return pkv::round256((size_t)pkv::kPrefixSlots * pkv::prefix_slot_floats(head_dim) * sizeof(float));
}

PKV_EXPORT int pkv_paged_attention_prefill(const void* q, int32_t q_dtype, int32_t num_seqs,
                                           int32_t num_tokens, int32_t num_q_heads,
                                           const int32_t* query_start, const void* k_cache,
                                           const void* v_cache, const pkv_cache_desc* cache,
                                           const int32_t* block_tables,
                                           int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, float scale,
                                           void* workspace, size_t workspace_bytes, void* out,
                                           hipStream_t stream) {
    if (num_tokens < 0 || query_start == nullptr) return PKV_ERR_INVALID_ARG;
    if (num_tokens == 0) {  // nothing to compute: q and out may be NULL
        const int rc0 = check_cache(cache);
        if (rc0 != PKV_OK) return rc0;
        return num_seqs > 0 && num_q_heads > 0 ? PKV_OK : PKV_ERR_INVALID_ARG;
    }
    // the same checks as decode (no workspace)
    pkv::DecodeArgs d;
    const int rc = decode_args(d, q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache,
                               block_tables, max_blocks_per_seq, context_lens, scale, 0,
                               false, nullptr, out, stream);
    if (rc != PKV_OK) return rc;
    if (pkv::prefill_task_bound(num_seqs, num_tokens, d.group, cache->num_kv_heads) +
            pkv::kPrefixTargetWorkgroups > INT32_MAX ||
        (int64_t)cache->num_kv_heads * (((int64_t)num_tokens * d.group) / 16 + num_seqs) > INT32_MAX)
        return PKV_ERR_UNSUPPORTED;
    if (workspace != nullptr && (((uintptr_t)workspace & 255u) != 0 ||
                                 workspace_bytes < pkv_prefill_workspace_bytes(cache->head_dim)))
        return PKV_ERR_WORKSPACE;
    pkv::PrefillArgs a{};
    a.q = q;
    a.q_dtype = q_dtype;
    a.kv_dtype = cache->dtype;
    a.num_seqs = num_seqs;
    a.num_tokens = num_tokens;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = cache->num_kv_heads;
    a.group = d.group;
    a.head_dim = cache->head_dim;
    a.num_blocks = cache->num_blocks;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.query_start = query_start;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.scale = scale;
    a.k_scale = cache->k_scale;
    a.v_scale = cache->v_scale;
    a.slots = static_cast<float*>(workspace);
    a.out = out;
    a.stream = stream;
    hipError_t err = pkv::launch_paged_prefill(a);
    return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

PKV_EXPORT int pkv_copy_blocks(void* k_cache, void* v_cache, const pkv_cache_desc* cache,
                               const int32_t* pairs, int32_t num_pairs, hipStream_t stream) {
    int rc = check_cache(cache);
    if (rc != PKV_OK) return rc;
    if (num_pairs < 0 || k_cache == nullptr || v_cache == nullptr ||
        (num_pairs > 0 && pairs == nullptr))
        return PKV_ERR_INVALID_ARG;
    if (!aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID_ARG;
    hipError_t err = pkv::launch_copy_blocks(k_cache, v_cache, elem_bytes(cache->dtype),
                                             cache->num_blocks, cache->num_kv_heads,
                                             cache->head_dim, pairs, num_pairs, stream);
    return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

PKV_EXPORT int pkv_debug_gather(const void* k_cache, const void* v_cache,
                                const pkv_cache_desc* cache, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t num_seqs, int32_t max_ctx, void* k_out, void* v_out,
                                hipStream_t stream) {
    int rc = check_cache(cache);
    if (rc != PKV_OK) return rc;
    if (num_seqs <= 0 || max_ctx < 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
    if (k_cache == nullptr || v_cache == nullptr || block_tables == nullptr ||
        context_lens == nullptr || k_out == nullptr || v_out == nullptr)
        return PKV_ERR_INVALID_ARG;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_out) || !aligned16(v_out))
        return PKV_ERR_INVALID_ARG;
    hipError_t err = pkv::launch_gather(k_cache, v_cache, elem_bytes(cache->dtype),
                                        cache->num_blocks, cache->num_kv_heads, cache->head_dim,
                                        block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                        max_ctx, k_out, v_out, stream);
    return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

PKV_EXPORT int pkv_stream_read(const void* src, size_t bytes, uint32_t* sink,
                               int32_t num_workgroups, hipStream_t stream) {
    if (src == nullptr || sink == nullptr || num_workgroups < 0) return PKV_ERR_INVALID_ARG;
    if (!aligned16(src) || bytes % 16 != 0 || ((uintptr_t)sink & 3u) != 0) return PKV_ERR_INVALID_ARG;
    if (bytes == 0) return PKV_OK;
    hipError_t err = pkv::launch_stream_read(src, bytes, sink, num_workgroups, stream);
    return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

// ---- allocation-free decode ------------------------------------------------
//
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc): the decode workspace is a
// static device array, one copy per GPU, held from the library's load on that
// GPU until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: only its device address, taken once per
// device with hipGetSymbolAddress, is ever passed on.

static __device__ __align__(256) uint8_t scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array (taken on the first
// call on that device).
int current_scratch(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
    if (dev < 0 || dev >= kMaxScratchDevices) return PKV_ERR_UNSUPPORTED;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
                return PKV_ERR_HIP;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return PKV_OK;
}

// Zero n int32 counters (a kernel rather than a memset, so the call can be
// captured in a HIP graph).
__global__ void clear_counters_kernel(int32_t* c, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        c[i] = 0;
}

}  // namespace

PKV_EXPORT int pkv_paged_attention_decode_noalloc(const void* q, int32_t q_dtype,
                                                  int32_t num_seqs, int32_t num_q_heads,
                                                  const void* k_cache, const void* v_cache,
                                                  const pkv_cache_desc* cache,
                                                  const int32_t* block_tables,
                                                  int32_t max_blocks_per_seq,
                                                  const int32_t* context_lens, float scale,
                                                  int32_t partition_size, int32_t num_workers,
                                                  void* out, hipStream_t stream) {
    pkv::DecodeArgs a;
    // the same checks as pkv_paged_attention_decode (the workspace is ours)
    const int rc = decode_args(a, q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache,
                               block_tables, max_blocks_per_seq, context_lens, scale, num_workers,
                               false, nullptr, out, stream);
    if (rc != PKV_OK) return rc;
    if (!partition_ok(partition_size)) return PKV_ERR_INVALID_ARG;
    const size_t need = pkv_decode_workspace_bytes(num_seqs, num_q_heads, cache->num_kv_heads,
                                                   cache->head_dim, max_blocks_per_seq,
                                                   partition_size, num_workers);
    if (need == 0) return PKV_ERR_INVALID_ARG;
    if (need > PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_TOO_LARGE;
    void* ws = nullptr;
    const int src = current_scratch(&ws);
    if (src != PKV_OK) return src;
    // the counters: the last bytes of the array, cleared for this call
    const size_t ctr_bytes = pkv::decode_counter_bytes(num_seqs, cache->num_kv_heads);
    int32_t* counters = reinterpret_cast<int32_t*>(
        static_cast<char*>(ws) + pkv::tail_offset(PKV_NOALLOC_SCRATCH_BYTES, ctr_bytes));
    const int n = (int)(ctr_bytes / sizeof(int32_t));
    hipLaunchKernelGGL(clear_counters_kernel, dim3((n + 255) / 256 < 64 ? (n + 255) / 256 : 64),
                       dim3(256), 0, stream, counters, n);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
    a.partition_size = partition_size;
    a.slots = static_cast<float*>(ws);
    a.counters = counters;
    hipError_t err = pkv::launch_paged_decode(a);
    return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
