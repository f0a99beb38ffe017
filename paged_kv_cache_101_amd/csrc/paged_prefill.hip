// paged_prefill.hip -- paged chunked-prefill attention for gfx950.
//
// What is computed (ttlab page, section 6, chunked prefill; section 4, the
// paged cache): each sequence brings a chunk of q_len new query tokens, the
// last q_len of its n cached tokens (their K/V already appended); token i of
// the chunk sits at position p = n - q_len + i and attends to positions
// 0..p of its own sequence, read through its block table.
//
// Unlike decode this is a real contraction: for one (sequence, KV head) the
// chunk's q_len * G query rows all meet the same K/V tiles. The kernel is
// tiled for the matrix cores accordingly:
//   * A workgroup of 4 waves owns 128 query rows of one (sequence, KV head),
//     stacked token-major (row = token * G + head), 32 per wave as two 16-row
//     MFMA column sets. Two workgroups share a CU (two waves per SIMD), and
//     their barriers are independent, so one's softmax and LDS reads overlap
//     the other's matrix work.
//   * The sequence's 16-token tiles stream through an LDS ring of two-tile
//     steps (four stages for 16-bit and fp8 tiles), issued three steps ahead
//     and moved from L2 straight into LDS by buffer loads (no registers).
//     Each wave reads a step's K and V operands from LDS once and applies
//     them to its 32 rows: a tile costs one L2 read per 128 rows.
//   * Per 16-row block: S^T = K . Q^T and O^T = V^T . P^T on MFMA, so the
//     query row is the MFMA column and every row statistic stays in the
//     row's lanes; online softmax in log2 units with a lazily moved maximum.
//     P^T . V contracts both tiles of a step in one 16x16x32 MFMA per 16
//     output columns. Tiles wholly before a row block's first position need
//     no mask; the diagonal tiles mask key k > p per row by select; steps
//     after the last position of all the wave's rows are skipped. A step's
//     products and weights form one straight-line stretch; only the
//     workgroup's last step (peeled off the loop) masks V.
//   * The steady steps (no select, no mask, no end check: most of them) run
//     in groups of four with fixed ring stages and a handful of scalar
//     instructions each: block ids eight at a time, tiles addressed by one
//     K and one V resource plus a 32-bit offset.
//   * Workgroup index -> (sequence, row tile, KV head) with the KV head fastest,
//     so the workgroups of one head land on one XCD (workgroups are dealt to
//     the 8 XCDs round-robin) and share its L2; within a sequence the row
//     tiles with the most keys start first.
//
// Batches with few row tiles (short chunks over long contexts) may split a
// row tile's keys into chunks, each a workgroup, when the caller passes a
// partial-slot workspace; chunk_merge_kernel then combines the partials.
//
// The same kernel in prefix mode is the prefix pass of the shared-prefix
// decode (see the end of this file): a prefix group's member sequences take
// the place of a chunk's tokens, every row sees every key of its part of the
// shared prefix, and the result is merged with the suffix pass's.
#include <type_traits>

#include "decode_wave.h"
#include "pkv_internal.h"
#include "pkv_tile.h"

namespace pkv {

namespace {

constexpr int kPrefillWaves = 4;                    // waves per workgroup
constexpr int kRowBlocks = 2;                       // 16-row blocks per wave
constexpr int kWaveRows = 16 * kRowBlocks;          // 32
constexpr int kGroupRows = kPrefillWaves * kWaveRows;  // 128
constexpr int kPrefillThreads = kPrefillWaves * kWave;

// s_waitcnt operand that waits for the vector-memory counter to reach n
// (expcnt and lgkmcnt left at their maxima; gfx9 encoding, vmcnt split
// over bits 3:0 and 15:14).
constexpr int vmcnt_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes, read at
// byte voff of the buffer, land at lds_base + l * 16 (lds_base is the same
// for the whole wave). The address is a uniform resource plus a 32-bit lane
// offset, so no 64-bit per-lane address is kept.
__device__ __forceinline__ void load_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint8_t* lds_base,
                                            uint32_t soff = 0) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16,
                                             voff, (int)soff, 0, 0);
}

// Eight consecutive block-table entries, read as one scalar load (a
// wave-uniform address; the loads of the scalar unit need only 4-byte
// alignment).
typedef int32_t i32x8_t __attribute__((ext_vector_type(8), aligned(4)));
__device__ __forceinline__ i32x8_t uniform_read8(const int32_t* p) {
    return *(const __attribute__((address_space(4))) i32x8_t*)p;
}

// Wait until at most n (0..16, wave-uniform; larger n waits for 16) of this
// wave's vector-memory operations are in flight: s_waitcnt takes its count
// as an immediate.
template <int N = 0>
__device__ __forceinline__ void wait_vmcnt_from(int n) {
    if constexpr (N >= 16) {
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(16));
    } else {
        if (n <= N) __builtin_amdgcn_s_waitcnt(vmcnt_wait(N));
        else wait_vmcnt_from<N + 1>(n);
    }
}
__device__ __forceinline__ void wait_vmcnt(int n) { wait_vmcnt_from<0>(n); }

// All waves of the workgroup reach this point, each with its LDS reads
// complete. A compiler barrier on both sides keeps memory accesses from
// moving across it; unlike __syncthreads() it does not wait for this wave's
// outstanding buffer loads into LDS (the ring's own waits count those).
// Waiting for the LDS reads matters because the compiler may move the
// products that consume a step's operands past the next step's barrier:
// the reads of a ring stage must be done before any wave, once past the
// barrier, issues the loads that refill that stage.
__device__ __forceinline__ void workgroup_barrier() {
    asm volatile("" ::: "memory");
    // lgkmcnt(0), vmcnt and expcnt left at their maxima (gfx9 encoding)
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

struct PrefillParams {
    const uint8_t* q;
    const uint8_t* k_cache;
    const uint8_t* v_cache;
    const int32_t* query_start;  // [S + 1]
    const int32_t* block_tables;
    const int32_t* context_lens;
    int num_seqs;
    int num_tokens;  // rows of q / out
    int num_q_heads;
    int num_kv_heads;
    int group;
    int num_blocks;
    int max_blocks_per_seq;
    float qk_scale_log2;
    float v_scale;
    void* out;
    // the prefix pass of the shared-prefix decode only
    int num_groups;
    const int32_t* group_starts;  // [num_groups + 1]
    const int32_t* group_prefix;  // [num_groups]
    float* slots;                 // [kPrefixSlots][prefix_slot_floats(D)]
    const float* res_o;           // suffix results [S][H_q][D] and [S][H_q]
    const float* res_lse;
    // prefix pass running beside the suffix pass: every group's partials go
    // to slots (none is merged with the suffix results here), and the chunk
    // count aims at pf_target workgroups (0: kPrefixTargetWorkgroups)
    int all_slots;
    int pf_target;
    // every tile's byte offset in the K and V caches fits 32 bits
    // (num_blocks * num_kv_heads * tile bytes < 2^32)
    int offsets32;
};

// Row tiles of kGroupRows rows of a sequence (0 for an invalid chunk).
__device__ __forceinline__ int row_tiles(const PrefillParams& p, int s) {
    const int a = p.query_start[s], b = p.query_start[s + 1];
    const int n = p.context_lens[s];
    if (a < 0 || b < a || b > p.num_tokens || n > p.max_blocks_per_seq * kBlock || b - a > n)
        return 0;
    return ((b - a) * p.group + kGroupRows - 1) / kGroupRows;
}

// Ring depth in two-tile steps: four when a step is at most 16 KiB, else three
// (two workgroups of a CU then fit in its LDS for every 16-bit and fp8 shape).
template <int KT, int D>
constexpr int ring_depth() {
    return 4 * kBlock * D * Elem<KT>::bytes <= 16384 ? 4 : 3;
}

// Waves per SIMD the attention kernel aims at: two workgroups of four waves
// share a CU when two rings fit its 160 KiB of LDS (every 16-bit and fp8
// shape, and float32 at d = 64); float32 at d = 128 (three 32 KiB stages)
// runs one workgroup per CU and may use every register.
template <int KT, int D>
constexpr int prefill_waves_per_simd() {
    return 2 * ring_depth<KT, D>() * 4 * kBlock * D * Elem<KT>::bytes <= 160 * 1024 ? 2 : 1;
}

// The 16-bit compute type of a query type (f32 queries never use it).
template <int QT>
struct Compute16 {
    typedef _Float16 E;
    typedef _Float16 V2 __attribute__((ext_vector_type(2)));
    typedef f16x8_t V8;
};
template <>
struct Compute16<PKV_BF16> {
    typedef __bf16 E;
    typedef __bf16 V2 __attribute__((ext_vector_type(2)));
    typedef bf16x8_t V8;
};

// The largest of its operands, NaN if any is NaN: no operand quieting is
// needed, and three operands take one instruction (v_maximum3_f32).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax(float a, float b, float c) { return vmax(vmax(a, b), c); }

// Four float results, elements idx .. idx + 3 of an output (idx a multiple of
// four, the base 16-byte aligned), in the output type.
template <int DT>
__device__ __forceinline__ void store4_as(void* base, size_t idx, float a, float b, float c, float d) {
    if constexpr (DT == PKV_F32) {
        *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(base) + idx) = f32x4_t{a, b, c, d};
    } else if constexpr (DT == PKV_F16) {
        const f16x4_t h = {(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
        *reinterpret_cast<u32x2_t*>(reinterpret_cast<_Float16*>(base) + idx) =
            __builtin_bit_cast(u32x2_t, h);
    } else {
        static_assert(DT == PKV_BF16, "output type");
        const u32x2_t w = {(uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16),
                           (uint32_t)f32_to_bf16_rne(c) | ((uint32_t)f32_to_bf16_rne(d) << 16)};
        *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(base) + idx) = w;
    }
}

// A prefill sequence's row tiles of 128 rows, 16-row blocks, and the key
// tiles of its first row tile (the fewest of any of its row tiles); zeros for
// an invalid or empty chunk.
__device__ __forceinline__ void prefill_seq_shape(const PrefillParams& p, int s, int& rts, int& rbs,
                                                  int& tmin) {
    rts = row_tiles(p, s);
    rbs = tmin = 0;
    if (rts == 0) return;
    const int q_len = p.query_start[s + 1] - p.query_start[s];
    const int rows = q_len * p.group;
    rbs = (rows + 15) / 16;
    tmin = (p.context_lens[s] - q_len + (min(rows, kGroupRows) - 1) / p.group) / kBlock + 1;
}

// The common chunk count for work whose rows fill rt_total row tiles of 128
// and rb_total row blocks of 16 (per KV head): about kPrefixTargetWorkgroups
// workgroups, and the chunked rows' 16-row partials within kPrefixSlots. The
// attention kernel and the merge launch derive it the same way.
__device__ __forceinline__ int prefix_chunks(int H, int rt_total, int rb_total, int target) {
    if (target <= 0) target = kPrefixTargetWorkgroups;
    const int per_chunk = H * rt_total;
    const int cg = per_chunk >= target ? 1 : (target + per_chunk - 1) / per_chunk;
    return min(cg, max(1, kPrefixSlots / (H * rb_total)));
}

}  // namespace

// PFX = false: chunked prefill, one (sequence, row tile, KV head) per
// workgroup, causal. PFX = true: the prefix pass of the shared-prefix decode
// -- one (prefix group, row tile, KV head, chunk of the prefix blocks) per
// workgroup, every row seeing every key of the chunk, the partial merged with
// the suffix results.
// One workgroup per task: task in [0, the grid's upper bound on tasks);
// workgroups past the last task return at once.
// FGM > 0 (prefix mode only): the shared-prefix call's single launch for both
// passes. Workgroups [0, suffix_wgs) run the suffix pass's worker waves, four
// to a workgroup (decode_wave in result mode, query heads padded to FGM), the
// rest the prefix pass's tasks (partials to slots). The two passes need
// nothing from each other, so they share the device from the start of the
// launch, with no second stream and no cross-stream events; the merge launch
// follows on the same stream. (On a second stream with a fork and a join, the
// merge started about 6 us after the suffix pass ended, and the suffix pass
// at times 11-14 us after the prefix pass began.)
template <int KT, int QT, int D, bool PFX, int FGM>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(prefill_waves_per_simd<KT, D>())))
void paged_prefill_kernel(PrefillParams p, DecodeParams dp, int suffix_wgs) {
    static_assert(FGM == 0 || PFX, "only the prefix pass shares a launch");
    int task_id = (int)blockIdx.x;
    if constexpr (FGM > 0) {
        if (task_id < suffix_wgs) {
            decode_wave<KT, QT, D, FGM, true, false>(
                dp, __builtin_amdgcn_readfirstlane(task_id * kPrefillWaves + wave_id()));
            return;
        }
        task_id -= suffix_wgs;
    }
    using TM = TileMath<KT, QT, D>;
    constexpr int NK = TM::NK, NV = TM::NV, NVL = TM::NVL, KW = TM::KW, VLW = TM::VLW;
    constexpr int VW = TM::VW;
    constexpr int KB = Elem<KT>::bytes;
    constexpr int QB = Elem<QT>::bytes;
    constexpr uint32_t kTileBytes = (uint32_t)kBlock * D * KB;
    constexpr int kRing = ring_depth<KT, D>();
    constexpr uint32_t kStepBytes = 4 * kTileBytes;
    constexpr bool kDirectV = (KB == 2);
    typedef typename Compute16<QT>::E E16;
    typedef typename Compute16<QT>::V2 V2;
    typedef typename Compute16<QT>::V8 V8;

    // kRing stages of two tiles' (K, V). 16-bit tiles: A's K, B's K, then the
    // V pieces of both alternating per 1 KiB (A's piece 0, B's piece 0, A's
    // piece 1, ...), so that the two chunks that make a pair of P . V
    // operands lie 1 KiB apart from one base. Other tiles: A's K, A's V, B's
    // K, B's V.
    __shared__ __attribute__((aligned(16))) uint8_t lds[kRing * kStepBytes];
    constexpr uint32_t kKTileB = kDirectV ? kTileBytes : 2 * kTileBytes;  // B's K in a stage

    const int lane = lane_id();
    const int wv = wave_id();
    const int S = p.num_seqs, H = p.num_kv_heads, G = p.group, Hq = p.num_q_heads;

    // ---- this workgroup's task ----
    // (row tiles of 128 rows stacked token-major, row = token * G + head; in
    // the prefix pass a group's members take the place of the chunk's tokens;
    // a row tile's keys may be split into chunks, each a workgroup of its own)
    int g = 0, q0 = 0, q_len = 0, n = 0, base_pos = 0, row_wg = 0, tiles = 0, tile0 = 0;
    size_t bt_row = 0;
    int pf_chunks = 1, pf_chunk = 0, rb_total = 0;  // prefix pass
    int64_t pf_task16 = 0;
    if constexpr (PFX) {
        const int mb = p.max_blocks_per_seq;
        const int ng = usable_groups(p.group_starts, p.group_prefix, p.num_groups, S, mb, lane);
        if (ng == 0) return;
        auto rows_of = [&](int j) {
            return p.group_prefix[j] > 0 ? (p.group_starts[j + 1] - p.group_starts[j]) * G : 0;
        };
        // 16-row blocks and 128-row tiles over the groups with a prefix
        int rt_total = 0;
        for (int base = 0; base < ng; base += kWave) {
            const int j = base + lane;
            const int rows = j < ng ? rows_of(j) : 0;
            rb_total += wave_sum_int((rows + 15) / 16);
            rt_total += wave_sum_int((rows + kGroupRows - 1) / kGroupRows);
        }
        if (rt_total == 0) return;
        const int cg = prefix_chunks(H, rt_total, rb_total, p.pf_target);
        // the group holding this workgroup (wave-uniform)
        const int task = task_id;
        int wg_before = 0;
        int64_t t16_before = 0;
        int jj = -1, local = 0;
        for (int base = 0; base < ng; base += kWave) {
            const int j = base + lane;
            const int rows = j < ng ? rows_of(j) : 0;
            const int cj = j < ng ? min(p.group_prefix[j], cg) : 0;
            const int rts = (rows + kGroupRows - 1) / kGroupRows, rbs = (rows + 15) / 16;
            const int wgs = H * rts * cj;
            const int incl = wave_inclusive_scan(wgs);
            const int tincl = wave_inclusive_scan(H * rbs * cj);
            const unsigned long long hit =
                __ballot(wgs > 0 && wg_before + incl - wgs <= task && task < wg_before + incl);
            if (hit) {
                const int L = __ffsll(hit) - 1;
                jj = base + L;
                local = task - wg_before - __builtin_amdgcn_readlane(incl - wgs, L);
                pf_task16 = t16_before + __builtin_amdgcn_readlane(tincl - H * rbs * cj, L);
                break;
            }
            wg_before += __builtin_amdgcn_readlane(incl, kWave - 1);
            t16_before += __builtin_amdgcn_readlane(tincl, kWave - 1);
        }
        if (jj < 0) return;  // the grid is an upper bound on the tasks
        const int pre = p.group_prefix[jj];
        pf_chunks = min(pre, cg);
        g = local % H;
        pf_chunk = (local / H) % pf_chunks;
        const int rt = local / H / pf_chunks;
        q0 = p.group_starts[jj];
        q_len = p.group_starts[jj + 1] - q0;
        tile0 = (int)((int64_t)pf_chunk * pre / pf_chunks);
        tiles = (int)((int64_t)(pf_chunk + 1) * pre / pf_chunks) - tile0;
        n = tiles * kBlock;  // every prefix block is full
        row_wg = rt * kGroupRows;
        bt_row = (size_t)q0 * mb;  // the group's blocks: its first member's table
    } else {
        // Sequences with few row tiles split each row tile's keys into chunks
        // when a partial-slot workspace is given (slots != nullptr).
        int cg = 1;
        if (p.slots != nullptr) {
            int rt_total = 0;
            for (int base = 0; base < S; base += kWave) {
                const int ss = base + lane;
                int rts = 0, rbs = 0, tmin = 0;
                if (ss < S) prefill_seq_shape(p, ss, rts, rbs, tmin);
                rt_total += wave_sum_int(rts);
                rb_total += wave_sum_int(rbs);
            }
            if (rt_total > 0) cg = prefix_chunks(H, rt_total, rb_total, p.pf_target);
        }
        const int task = task_id;
        int s = -1, local = 0;
        int before = 0;
        int64_t t16_before = 0;
        for (int base = 0; base < S; base += kWave) {
            const int ss = base + lane;
            int rts = 0, rbs = 0, tmin = 0;
            if (ss < S) prefill_seq_shape(p, ss, rts, rbs, tmin);
            const int cs = min(cg, max(tmin, 1));
            const int cnt = rts * H * cs;
            const int incl = wave_inclusive_scan(cnt);
            const int tincl = wave_inclusive_scan(H * rbs * cs);
            const unsigned long long hit = __ballot(cnt > 0 && before + incl - cnt <= task &&
                                                    task < before + incl);
            if (hit) {
                const int L = __ffsll(hit) - 1;
                s = base + L;
                local = task - before - __builtin_amdgcn_readlane(incl - cnt, L);
                pf_task16 = t16_before + __builtin_amdgcn_readlane(tincl - H * rbs * cs, L);
                pf_chunks = __builtin_amdgcn_readlane(cs, L);
                break;
            }
            before += __builtin_amdgcn_readlane(incl, kWave - 1);
            t16_before += __builtin_amdgcn_readlane(tincl, kWave - 1);
        }
        if (s < 0) return;  // the grid is an upper bound on the tasks
        g = local % H;
        pf_chunk = (local / H) % pf_chunks;
        const int rt = row_tiles(p, s) - 1 - local / H / pf_chunks;  // the longest row tiles first
        q0 = p.query_start[s];
        q_len = p.query_start[s + 1] - q0;
        n = p.context_lens[s];
        base_pos = n - q_len;  // position of the chunk's first token
        row_wg = rt * kGroupRows;
        const int last_row = min(q_len * G, row_wg + kGroupRows) - 1;
        const int tiles_rt = (base_pos + last_row / G) / kBlock + 1;  // keys 0 .. last position
        // this workgroup's chunk of them; positions are counted from its first key
        tile0 = (int)((int64_t)pf_chunk * tiles_rt / pf_chunks);
        tiles = (int)((int64_t)(pf_chunk + 1) * tiles_rt / pf_chunks) - tile0;
        base_pos -= tile0 * kBlock;
        n -= tile0 * kBlock;
        bt_row = (size_t)s * p.max_blocks_per_seq;
    }
    const int nrows = q_len * G;
    const int steps = (tiles + 1) / 2;
    const int key_end = tiles * kBlock - 1;  // the chunk's last key (positions from its first)

    // The score scale in log2 units, made non-negative: a negative scale
    // flips the sign of q instead (exact), so that the running maximum can be
    // taken on the raw scores.
    const float c = fabsf(p.qk_scale_log2);
    const uint32_t q_flip = p.qk_scale_log2 < 0.f ? (QB == 4 ? 0x80000000u : 0x80008000u) : 0u;

    // ---- per lane: its query row (column t of the MFMA tiles) in each row block ----
    const int t = lane & 15;
    const int g4 = lane >> 4;
    const int row_w = row_wg + wv * kWaveRows;
    typename TM::Q q[kRowBlocks];
    int pos[kRowBlocks];  // position of this lane's row (rows past the chunk: the last one)
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
        const int row = row_w + rb * 16 + t;
        const bool ok = row < nrows;
        const int tok = ok ? row / G : q_len - 1;
        // A row sees keys up to its position, and only those of this
        // workgroup's chunk of keys: as if it sat at most at the chunk's last
        // key (so a stand-in second tile past the chunk is masked). In the
        // prefix pass every row sees every key of the chunk.
        pos[rb] = PFX ? key_end : min(base_pos + tok, key_end);
        const int h = g * G + (ok ? row % G : 0);
        TM::load_q(q[rb], p.q + ((size_t)(q0 + tok) * Hq + h) * D * QB, ok, g4);
#pragma unroll
        for (int i = 0; i < NK; ++i)
#pragma unroll
            for (int x = 0; x < TM::QW; ++x) q[rb].w[i][x] ^= q_flip;
    }
    // row-block extents (wave-uniform): first and last valid position
    int rb_first[kRowBlocks], rb_last[kRowBlocks];
    int wave_last = -1;  // the last position any row of the wave has
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
        const int r0 = row_w + rb * 16;
        const int r1 = min(nrows, r0 + 16) - 1;
        rb_first[rb] = r0 < nrows ? (PFX ? key_end : min(base_pos + r0 / G, key_end)) : INT32_MAX;
        rb_last[rb] = r0 < nrows ? (PFX ? key_end : min(base_pos + r1 / G, key_end)) : -1;
        wave_last = max(wave_last, rb_last[rb]);
    }
    // A step needs the causal select for row block rb once its last key
    // passes sel_from[rb]; a block with no valid row always takes it, so its
    // stand-in rows never score keys past their position.
    int sel_from[kRowBlocks];
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) sel_from[rb] = rb_last[rb] >= 0 ? rb_first[rb] : -1;

    // ---- the tile stream: an LDS ring of two-tile steps, filled by direct loads ----
    // Step sp (tiles 2 sp and 2 sp + 1) goes to ring stage sp % kRing. It is
    // moved from L2 straight into LDS (no registers) in 1 KiB pieces, 16 bytes
    // per lane, piece c carried by wave c % 4, kRing - 1 steps ahead of the
    // step whose P . V is computed. A wave waits for its own loads (the
    // counter counts them in issue order), then the barrier makes every
    // wave's pieces visible. A tile past the last one reads the null block.
    constexpr int kPieces = 2 * (int)kTileBytes / 1024;  // of one tile: its K, then its V
    constexpr int kStepPieces = 2 * kPieces;
    constexpr int kWavePieces = (kStepPieces + kPrefillWaves - 1) / kPrefillWaves;  // at most
    static_assert(kTileBytes % 1024 == 0, "piece split");
    static_assert((kRing - 2) * kWavePieces <= 16, "wait count");
    // V pieces are stored permuted so that the V operand reads are
    // conflict-free: a lane's V load i (tokens 4 * g4 .. + 3 of its element
    // columns, kVChunks 16-byte chunks) sits at chunk 4 * t + g4 (times
    // kVChunks) of its region of the tile, and the piece's lane L fetches the
    // chunk that the lane reading 16-byte slot L needs. Float32 tiles: lane
    // (t, g4) reads slot 16 g4 + t. 16-bit tiles: slot v_slot(t, g4) below,
    // read as two 8-byte halves. fp8 V loads are 8 bytes per lane and are
    // stored as they are.
    constexpr int kVChunks = VLW / 4;
    auto v_piece_src = [&](int pc) -> uint32_t {
        if constexpr (kDirectV) {
            // the inverse of v_slot: slot L = 16 g4 + r is read by lane (tl, g4)
            const int g4l = lane >> 4, r = lane & 15;
            const int tl = (r & 7) + 8 * ((r >> 3) ^ (g4l & 1));
            return (uint32_t)(pc * 1024 + (4 * tl + g4l) * 16);
        } else if constexpr (kVChunks > 0) {
            const int i = pc / kVChunks, h = pc % kVChunks;
            const int sigma = 4 * (lane & 15) + (lane >> 4);  // 4 * t + g4 of reading lane L
            return (uint32_t)(i * 1024 * kVChunks + (kVChunks * sigma + h) * 16);
        } else {
            return (uint32_t)pc * 1024 + (uint32_t)lane * 16;
        }
    };
    // What this wave carries of every step (the same pieces each step): the
    // cache and this lane's 16 bytes inside the tile, the tile (A or B), and
    // the piece's place in the stage. Fixed before the loop, so that issuing
    // a step takes no look-up of the kernel arguments.
    uint32_t pc_src[kWavePieces];  // this lane's offset in the tile (per lane)
    uint32_t pc_dst[kWavePieces];
    bool pc_b[kWavePieces], pc_v[kWavePieces];
    bool pc_ok[kWavePieces];  // the wave carries piece i (the last may be absent)
    const int my_pieces = (kStepPieces - wv + kPrefillWaves - 1) / kPrefillWaves;
    // When a tile's K (and its V) splits into a multiple of four pieces, every
    // wave carries the same roles in the same order (piece i of the wave:
    // tile (4 i) / kPieces, K or V by (4 i) % kPieces), known at compile
    // time, so issuing a step selects no resource at run time.
    constexpr bool kFixedRoles = kPieces % (2 * kPrefillWaves) == 0;
    auto fixed_b = [](int i) { return (kPrefillWaves * i) / kPieces == 1; };
    auto fixed_v = [](int i) { return (kPrefillWaves * i) % kPieces >= kPieces / 2; };
#pragma unroll
    for (int i = 0; i < kWavePieces; ++i) {
        const int c2 = min(wv + i * kPrefillWaves, kStepPieces - 1);
        pc_ok[i] = wv + i * kPrefillWaves < kStepPieces;
        const int th = c2 / kPieces;  // 0: tile A, 1: tile B
        const int cc = c2 % kPieces;
        const bool is_v = cc >= kPieces / 2;
        const int pc = is_v ? cc - kPieces / 2 : cc;
        pc_src[i] = is_v ? v_piece_src(pc) : (uint32_t)pc * 1024 + (uint32_t)lane * 16;
        pc_v[i] = is_v;
        if constexpr (kDirectV)
            pc_dst[i] = is_v ? 2 * kTileBytes + (uint32_t)(2 * pc + th) * 1024
                             : (uint32_t)th * kTileBytes + (uint32_t)pc * 1024;
        else
            pc_dst[i] = (uint32_t)th * 2 * kTileBytes + (is_v ? kTileBytes : 0) + (uint32_t)pc * 1024;
        pc_b[i] = th == 1;
    }
    bool bad = false;
    // Block-table entries of step sp's two tiles as read (0, the null block,
    // past the last tile). They are read an iteration before the step is
    // issued and checked only then, so the scalar loads are not waited for
    // at once.
    auto step_ids = [&](int sp, int& ia, int& ib) {
        ia = 2 * sp < tiles ? uniform_read(p.block_tables, bt_row + tile0 + 2 * sp) : 0;
        ib = 2 * sp + 1 < tiles ? uniform_read(p.block_tables, bt_row + tile0 + 2 * sp + 1) : 0;
    };
    auto checked = [&](int id) -> int {
        if ((uint32_t)id >= (uint32_t)p.num_blocks) {  // negative ids too
            bad = true;  // its rows become NaN; the null block is read instead
            return 0;
        }
        return id;
    };
    // Byte offset of tile (block id, KV head g): the product (id * H + g)
    // fits 32 bits (num_blocks * H < 2^31); the byte offset may not.
    auto tile_bytes_at = [&](int id) -> size_t {
        return (size_t)(uint32_t)(id * H + g) * kTileBytes;
    };
    auto issue = [&](int sp, int ia, int ib) {
        const uint32_t st = (uint32_t)(sp % kRing) * kStepBytes;
        const size_t off_a = tile_bytes_at(checked(ia));
        const size_t off_b = tile_bytes_at(checked(ib));
        const __amdgpu_buffer_rsrc_t rka = make_rsrc(p.k_cache + off_a, kTileBytes);
        const __amdgpu_buffer_rsrc_t rva = make_rsrc(p.v_cache + off_a, kTileBytes);
        const __amdgpu_buffer_rsrc_t rkb = make_rsrc(p.k_cache + off_b, kTileBytes);
        const __amdgpu_buffer_rsrc_t rvb = make_rsrc(p.v_cache + off_b, kTileBytes);
#pragma unroll
        for (int i = 0; i < kWavePieces; ++i) {
            if constexpr (kFixedRoles) {
                load_to_lds(fixed_v(i) ? (fixed_b(i) ? rvb : rva) : (fixed_b(i) ? rkb : rka),
                            pc_src[i], lds + st + pc_dst[i]);
            } else if (pc_ok[i]) {
                load_to_lds(pc_v[i] ? (pc_b[i] ? rvb : rva) : (pc_b[i] ? rkb : rka), pc_src[i],
                            lds + st + pc_dst[i]);
            }
        }
    };
    // wait until at most `later` steps' loads of this wave are in flight
    auto wait_steps = [&](int later) {
        if constexpr (kFixedRoles) {
            // the steady state (kRing - 3 steps still in flight) as one immediate
            if (later == kRing - 3) __builtin_amdgcn_s_waitcnt(vmcnt_wait((kRing - 3) * kWavePieces));
            else wait_vmcnt(later * kWavePieces);
        } else {
            wait_vmcnt(later * my_pieces);
        }
    };

    const uint32_t k_off = (uint32_t)((g4 * kBlock + t) * 8 * KB);
    const uint32_t v_off = (uint32_t)((t * 4 + g4) * 8 * KB);
    const int x16 = (lane ^ 16) << 2, x32 = (lane ^ 32) << 2;

    auto read_k = [&](uint32_t base, uint32_t (&kr)[NK][KW]) {
#pragma unroll
        for (int i = 0; i < NK; ++i)
#pragma unroll
            for (int x = 0; x < KW; ++x)
                kr[i][x] = reinterpret_cast<const uint32_t*>(lds + base + k_off + i * 4 * kBlock * 8 * KB)[x];
    };
    auto read_v = [&](uint32_t base, uint32_t (&vr)[NVL][VLW]) {
        if constexpr (kVChunks > 0) {
            // the permuted store: this lane's 16-byte chunks sit at lane * 16
#pragma unroll
            for (int i = 0; i < NVL; ++i)
#pragma unroll
                for (int h = 0; h < kVChunks; ++h)
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        vr[i][4 * h + x] = reinterpret_cast<const uint32_t*>(
                            lds + base + (kVChunks * i + h) * 1024 + lane * 16)[x];
        } else {
#pragma unroll
            for (int i = 0; i < NVL; ++i)
#pragma unroll
                for (int x = 0; x < VLW; ++x)
                    vr[i][x] = reinterpret_cast<const uint32_t*>(lds + base + v_off + i * 32 * kBlock * KB)[x];
        }
    };
    // Running state per row block, for this lane's row t: the maximum m (log2
    // units, scaled), the lane's part of the weight sum, and O^T: o[rb][j]
    // holds elements 16 j + 4 g4 + r of row t (O^T = V^T P^T puts the query
    // row in the MFMA column, so every row statistic stays in its lanes).
    // m_use is the maximum the weights subtract: m, or 0 while m is -inf (a
    // row that has seen no key yet), so -inf - (-inf) never arises.
    float m_run[kRowBlocks], m_use[kRowBlocks], l_run[kRowBlocks];
    f32x4_t o[kRowBlocks][NV];
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
        m_run[rb] = -INFINITY;
        m_use[rb] = 0.f;
        l_run[rb] = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) o[rb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // S^T of both tiles of a stage for every row block: the NK-slab chains of
    // the four (tile, row block) pairs interleaved.
    auto qk_products = [&](const uint32_t (&kr)[2][NK][KW], f32x4_t (&sc)[2][kRowBlocks]) {
#pragma unroll
        for (int th = 0; th < 2; ++th)
#pragma unroll
            for (int rb = 0; rb < kRowBlocks; ++rb) sc[th][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NK; ++i)
#pragma unroll
            for (int th = 0; th < 2; ++th)
#pragma unroll
                for (int rb = 0; rb < kRowBlocks; ++rb) {
                    if constexpr (TM::kF32) {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            sc[th][rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                __builtin_bit_cast(float, kr[th][i][e]),
                                __builtin_bit_cast(float, q[rb].w[i][e]), sc[th][rb], 0, 0, 0);
                    } else if constexpr (QT == PKV_F16) {
                        const u32x4_t qu = {q[rb].w[i][0], q[rb].w[i][1], q[rb].w[i][2], q[rb].w[i][3]};
                        sc[th][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            TM::template k_operand<f16x8_t>(kr[th][i]), __builtin_bit_cast(f16x8_t, qu),
                            sc[th][rb], 0, 0, 0);
                    } else {
                        const u32x4_t qu = {q[rb].w[i][0], q[rb].w[i][1], q[rb].w[i][2], q[rb].w[i][3]};
                        sc[th][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            TM::template k_operand<bf16x8_t>(kr[th][i]),
                            __builtin_bit_cast(bf16x8_t, qu), sc[th][rb], 0, 0, 0);
                    }
                }
    };
    auto scores = [&](uint32_t st, f32x4_t (&sc)[2][kRowBlocks]) {
        uint32_t kr[2][NK][KW];
        read_k(st, kr[0]);
        read_k(st + kKTileB, kr[1]);
        qk_products(kr, sc);
    };
    // V of the step in stage st: for 16-bit caches the P . V operands
    // themselves (operand j = tile A's 4 tokens of element column 16 j + t,
    // then tile B's), else the loads. A lane's 16-byte chunk of each tile
    // holds two operands' halves (element columns 32 i + t and 32 i + 16 + t),
    // read as two 8-byte halves, each straight into its operand. The lanes of
    // columns t >= 8 take the halves the other way round (their operand 2 i
    // is column 32 i + 16 + t, and o[.][2 i], o[.][2 i + 1] trade places for
    // those output elements until the loop ends), and the chunk of lane
    // (t, g4) sits at slot v_slot(t, g4): together these make both 8-byte
    // reads conflict-free (any 16 or 32 consecutive lanes hit distinct
    // banks). Reading the chunk whole and pairing the halves in registers
    // took about 24 register moves per step; reading the halves at a 16-byte
    // lane stride had two-way bank conflicts.
    const int v_first = (t >> 3) * 8;  // byte of the chunk that operand 2 i takes
    const uint32_t v_slot = (uint32_t)(16 * g4 + (t & 7) + 8 * ((g4 & 1) ^ (t >> 3))) * 16;
    auto read_vops = [&](uint32_t st, u32x4_t (&vop)[NV], uint32_t (&va)[NVL][VLW],
                         uint32_t (&vb)[NVL][VLW]) {
        if constexpr (kDirectV) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const uint8_t* la = lds + st + 2 * kTileBytes + v_slot + (hh == 0 ? v_first : 8 - v_first);
#pragma unroll
                for (int i = 0; i < NVL; ++i) {
                    const u32x2_t a2 = *reinterpret_cast<const u32x2_t*>(la + 2 * i * 1024);
                    const u32x2_t b2 = *reinterpret_cast<const u32x2_t*>(la + (2 * i + 1) * 1024);
                    vop[2 * i + hh] = __builtin_shufflevector(a2, b2, 0, 1, 2, 3);
                }
            }
        } else {
            read_v(st + kTileBytes, va);
            read_v(st + 3 * kTileBytes, vb);
        }
    };
    // Zero the V elements of keys that no row sees: na and nb live keys
    // among this lane's four of tile A and of tile B.
    auto mask_vops = [&](int na, int nb, u32x4_t (&vop)[NV], uint32_t (&va)[NVL][VLW],
                         uint32_t (&vb)[NVL][VLW]) {
        if constexpr (kDirectV) {
            // dword d of a lane's four tokens holds tokens 2 d and 2 d + 1
            auto m2 = [](int live, int d) -> uint32_t {
                return live >= 2 * d + 2 ? ~0u : live == 2 * d + 1 ? 0xFFFFu : 0u;
            };
            const u32x4_t m = {m2(na, 0), m2(na, 1), m2(nb, 0), m2(nb, 1)};
#pragma unroll
            for (int j = 0; j < NV; ++j) vop[j] &= m;
        } else {
            TM::mask_v(va, na);
            TM::mask_v(vb, nb);
        }
    };
    // The largest of a row block's eight scores held by this lane.
    auto max8 = [](const float (&x)[8]) -> float {
        return vmax(vmax(vmax(x[0], x[1]), x[2]), vmax(vmax(x[3], x[4]), x[5]), vmax(x[6], x[7]));
    };
    // Move row block rb's running maximum when a score (this lane's largest:
    // xm, raw) exceeds it by more than the lazy margin in any lane.
    auto rescale = [&](int rb, float xm) {
        if (__any(xm * c > m_run[rb] + kLazyRescale)) {
            float tm = vmax(xm, lane_fetch(x16, xm));
            tm = vmax(tm, lane_fetch(x32, tm));
            const float mn = vmax(m_run[rb], tm * c);
            // a row that has seen no key yet (a chunk that starts past it)
            // keeps its zero sums
            const float cf = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - mn);
            l_run[rb] *= cf;
#pragma unroll
            for (int j = 0; j < NV; ++j) o[rb][j] *= cf;
            m_run[rb] = mn;
            m_use[rb] = mn == -INFINITY ? 0.f : mn;
        }
    };
    // The weights of a row block's eight raw scores against the maximum m,
    // rounded to the 16-bit type in pairs and packed as the P^T operand;
    // l_run gains their sum as rounded (dot products with ones).
    auto weights16 = [&](int rb, const float (&x)[8], float m) -> V8 {
        V2 h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            h[i] = V2{(E16)__builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * i], c, -m)),
                      (E16)__builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * i + 1], c, -m))};
        const V2 one = {(E16)1.f, (E16)1.f};
        float l = l_run[rb];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (QT == PKV_F16) l = __builtin_amdgcn_fdot2(h[i], one, l, false);
            else l = __builtin_amdgcn_fdot2_f32_bf16(h[i], one, l, false);
        }
        l_run[rb] = l;
        return __builtin_shufflevector(__builtin_shufflevector(h[0], h[1], 0, 1, 2, 3),
                                       __builtin_shufflevector(h[2], h[3], 0, 1, 2, 3), 0, 1, 2, 3, 4,
                                       5, 6, 7);
    };
    // O^T += V^T P^T for row block rb (16-bit operands).
    auto pv16 = [&](int rb, V8 pk, const u32x4_t (&vop)[NV], const uint32_t (&va)[NVL][VLW],
                    const uint32_t (&vb)[NVL][VLW]) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            V8 vj;
            if constexpr (kDirectV) vj = __builtin_bit_cast(V8, vop[j]);
            else vj = TM::template v_operand<V8>(va, vb, j);
            if constexpr (QT == PKV_F16)
                o[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vj, pk, o[rb][j], 0, 0, 0);
            else
                o[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vj, pk, o[rb][j], 0, 0, 0);
        }
    };

    // ---- the steady steps ----
    // Most steps need no causal select, no mask and no end-of-chunk check.
    // For 16-bit 128-wide tiles (four ring stages, every wave carrying the
    // same pieces) over caches whose tile offsets fit 32 bits, they run in
    // groups of four with the ring stages fixed at compile time, the block
    // ids of four steps read by one scalar load, and every tile addressed
    // through one K and one V resource plus a 32-bit offset: a handful of
    // scalar instructions per step instead of the general step's checks,
    // look-ups and resource set-up. The block ids of the workgroup's chunk
    // are checked once, here (any id out of range: the general steps, which
    // flag the rows, take the whole chunk).
    constexpr bool kQuadShape = kDirectV && kFixedRoles && kRing == 4;
    int quads = 0;  // groups of four steady steps, from step 0
    if constexpr (kQuadShape) {
        if (p.offsets32) {
            bool ids_ok = true;
            for (int b0 = 0; b0 < tiles && ids_ok; b0 += kWave) {
                const int i = b0 + lane;
                const int id = i < tiles ? p.block_tables[bt_row + tile0 + i] : 0;
                ids_ok = !__any((uint32_t)id >= (uint32_t)p.num_blocks);
            }
            int min_sel = INT32_MAX;
#pragma unroll
            for (int rb = 0; rb < kRowBlocks; ++rb) min_sel = min(min_sel, sel_from[rb]);
            // step sp needs no select while 32 sp + 31 <= min_sel, and the
            // step it issues (sp + 3) has both tiles while sp + 3 <= steps - 2
            const int sel_end = min_sel < 2 * kBlock - 1 ? 0 : (min_sel - (2 * kBlock - 1)) / (2 * kBlock) + 1;
            if (ids_ok) quads = max(0, min(sel_end, steps - kRing)) / 4;
        }
    }
    const __amdgpu_buffer_rsrc_t rk_all = make_rsrc(p.k_cache, 0xFFFFFFFFu);
    const __amdgpu_buffer_rsrc_t rv_all = make_rsrc(p.v_cache, 0xFFFFFFFFu);
    const uint32_t tile_mul = (uint32_t)H * kTileBytes, tile_add = (uint32_t)g * kTileBytes;
    auto issue_quad = [&](uint32_t st, int ia, int ib) {
        const uint32_t oa = (uint32_t)ia * tile_mul + tile_add, ob = (uint32_t)ib * tile_mul + tile_add;
#pragma unroll
        for (int i = 0; i < kWavePieces; ++i)
            load_to_lds(fixed_v(i) ? rv_all : rk_all, pc_src[i], lds + st + pc_dst[i], fixed_b(i) ? ob : oa);
    };

    for (int sp = 0; sp < kRing - 1 && sp < steps; ++sp) {
        int ia, ib;
        step_ids(sp, ia, ib);
        issue(sp, ia, ib);
    }
    wait_steps(min(kRing - 2, steps - 1));
    workgroup_barrier();
    // The scores of the step being computed and of the next one alternate
    // between two register sets (the loops take two or four steps at a
    // time), so the next step's products never have to be copied into the
    // current step's set.
    f32x4_t s_cur[2][kRowBlocks], s_alt[2][kRowBlocks];
    scores(0, s_cur);
    int nia = 0, nib = 0;  // block ids of the next step a general step issues

    // One step of the loop. kLast: the workgroup's last step, the only one
    // with no next step, and the only one whose keys can reach past n (the
    // unused rows of a sequence's last block) or whose tile B can be absent
    // (an odd tile count): chunk lengths put every other step's 32 keys
    // below n.
    // kQ >= 0: a steady step, the kQ-th of its group of four (ring stage
    // kQ; ia, ib: the block ids of the step it issues); -1: a general step.
    auto step = [&](auto last_c, auto quad_c, int sp, f32x4_t (&s_now)[2][kRowBlocks],
                    f32x4_t (&s_nxt)[2][kRowBlocks], int ia, int ib) __attribute__((always_inline)) {
            constexpr bool kLast = decltype(last_c)::value;
            constexpr int kQ = decltype(quad_c)::value;
            constexpr bool kSteady = kQ >= 0;
            if constexpr (kSteady) {
                __builtin_amdgcn_s_waitcnt(vmcnt_wait((kRing - 3) * kWavePieces));
                workgroup_barrier();
                issue_quad((uint32_t)((kQ + kRing - 1) % kRing) * kStepBytes, ia, ib);
            } else if constexpr (!kLast) {
                // step sp + 1 in LDS for every wave; stage (sp - 1) % kRing free
                wait_steps(min(kRing - 3, steps - 2 - sp));
                workgroup_barrier();
                if (sp + kRing - 1 < steps) issue(sp + kRing - 1, nia, nib);
            }
            const uint32_t st = kSteady ? (uint32_t)kQ * kStepBytes : (uint32_t)(sp % kRing) * kStepBytes;
            const uint32_t st_next = kSteady ? (uint32_t)((kQ + 1) % kRing) * kStepBytes
                                             : (uint32_t)((sp + 1) % kRing) * kStepBytes;
            const int key0 = 2 * sp * kBlock;  // first key of tile A; tile B starts at key0 + 16
            const bool has_b = 2 * sp + 1 < tiles;
            if constexpr (!TM::kF32) {
                if (kSteady || wave_last >= key0) {  // else every row of the wave is complete
                    // The next step's K reads and this step's V reads (their
                    // LDS latency passes under the maximum), this step's
                    // maximum (the rare rescale first), then one straight-line
                    // stretch (no branch:
                    // the compiler may overlap the next step's QK products with
                    // this step's weights, and the accumulators have one
                    // definition per step): QK products, weights and P . V.
                    // Diagonal steps replace the scores of keys past a row's
                    // position by -inf. On the last step, keys at or past n and
                    // an absent tile B (past the workgroup's last tile, which
                    // the causal limit, not n, can end) are seen by no row:
                    // their V elements are zeroed too, so that whatever those
                    // rows hold cannot reach P . V.
                    uint32_t kr[2][NK][KW];
                    if constexpr (!kLast) {
                        read_k(st_next, kr[0]);
                        read_k(st_next + kKTileB, kr[1]);
                    }
                    u32x4_t vop[NV];
                    uint32_t va[NVL][VLW], vb[NVL][VLW];
                    read_vops(st, vop, va, vb);
                    float x[kRowBlocks][8], xm[kRowBlocks];
                    bool trig = false;
#pragma unroll
                    for (int rb = 0; rb < kRowBlocks; ++rb) {
                        // raw scores: tile A keys key0 + 4 g4 + e, tile B keys key0 + 16 + 4 g4 + e
                        // (selected in place, so that they keep their registers)
                        if (!kSteady && key0 + 2 * kBlock - 1 > sel_from[rb]) {
                            const int lim = pos[rb] - key0 - 4 * g4;  // visible: key offsets up to lim
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                s_now[0][rb][e] = e <= lim ? s_now[0][rb][e] : -INFINITY;
                                s_now[1][rb][e] = kBlock + e <= lim ? s_now[1][rb][e] : -INFINITY;
                            }
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            x[rb][e] = s_now[0][rb][e];
                            x[rb][4 + e] = s_now[1][rb][e];
                        }
                        xm[rb] = max8(x[rb]);
                        trig = trig || xm[rb] * c > m_run[rb] + kLazyRescale;
                    }
                    if (__any(trig)) {
#pragma unroll
                        for (int rb = 0; rb < kRowBlocks; ++rb) rescale(rb, xm[rb]);
                    }
                    if constexpr (!kLast) qk_products(kr, s_nxt);
                    V8 pk[kRowBlocks];
#pragma unroll
                    for (int rb = 0; rb < kRowBlocks; ++rb) pk[rb] = weights16(rb, x[rb], m_use[rb]);
                    if constexpr (kLast) {
                        const int na = n - key0 - 4 * g4;        // live keys among this lane's four of tile A
                        const int nb = has_b ? na - kBlock : 0;  // and of tile B (the null block: none)
                        mask_vops(na, nb, vop, va, vb);
                    }
#pragma unroll
                    for (int rb = 0; rb < kRowBlocks; ++rb) pv16(rb, pk[rb], vop, va, vb);
                }
            } else if (wave_last >= key0) {  // else every row of the wave is complete
                // float32: this step's softmax and P . V, then the next step's
                // scores. Keys at or past n and a tile B past the workgroup's last
                // tile are seen by no row: their V elements are zeroed and their
                // scores excluded by select.
                u32x4_t vop[NV];
                uint32_t va[NVL][VLW], vb[NVL][VLW];
                read_vops(st, vop, va, vb);
                const int na = n - key0 - 4 * g4;          // live keys among this lane's four of tile A
                const int nb = has_b ? na - kBlock : 0;  // and of tile B (the null block: none)
                if (kLast) mask_vops(na, nb, vop, va, vb);
#pragma unroll
                for (int rb = 0; rb < kRowBlocks; ++rb) {
                    if (rb_last[rb] < key0) continue;  // no row of the block sees this step
                    // raw scores: tile A keys key0 + 4 g4 + e, tile B keys key0 + 16 + 4 g4 + e
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[e] = s_now[0][rb][e];
                        x[4 + e] = s_now[1][rb][e];
                    }
                    if (key0 + 2 * kBlock - 1 > rb_first[rb]) {  // a diagonal step: causal select
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            x[e] = key0 + 4 * g4 + e <= pos[rb] ? x[e] : -INFINITY;
                            x[4 + e] = key0 + kBlock + 4 * g4 + e <= pos[rb] ? x[4 + e] : -INFINITY;
                        }
                    }
                    rescale(rb, max8(x));
                    const float m = m_use[rb];
                    float pw[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) pw[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], c, -m));
                    // O^T += V^T P^T per tile on 16x16x4: k index = key 4 g4 + kk
#pragma unroll
                    for (int j = 0; j < NV; ++j)
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) {
                            o[rb][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                __builtin_bit_cast(float, va[j / 2][(j % 2) * VW + kk]), pw[kk],
                                o[rb][j], 0, 0, 0);
                            o[rb][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                __builtin_bit_cast(float, vb[j / 2][(j % 2) * VW + kk]), pw[4 + kk],
                                o[rb][j], 0, 0, 0);
                        }
                    l_run[rb] += ((pw[0] + pw[1]) + (pw[2] + pw[3])) + ((pw[4] + pw[5]) + (pw[6] + pw[7]));
                }
                if (!kLast && wave_last >= key0 + 2 * kBlock) scores(st_next, s_nxt);
            }
            if constexpr (!kLast && !kSteady)
                if (sp + kRing < steps) step_ids(sp + kRing, nia, nib);
    };
    using General = std::integral_constant<int, -1>;
    int sp = 0;
    if constexpr (kQuadShape) {
        if (quads > 0) {
            // the ids of the steps issued by group q: tiles 8 q + 6 .. 8 q + 13
            const int32_t* idp = p.block_tables + bt_row + tile0 + 2 * (kRing - 1);
            i32x8_t ids = uniform_read8(idp);
            for (int q = 0; q < quads; ++q, sp += 4) {
                i32x8_t nxt = ids;
                if (q + 1 < quads) nxt = uniform_read8(idp + 8 * (q + 1));
                step(std::false_type{}, std::integral_constant<int, 0>{}, sp, s_cur, s_alt, ids[0], ids[1]);
                step(std::false_type{}, std::integral_constant<int, 1>{}, sp + 1, s_alt, s_cur, ids[2], ids[3]);
                step(std::false_type{}, std::integral_constant<int, 2>{}, sp + 2, s_cur, s_alt, ids[4], ids[5]);
                step(std::false_type{}, std::integral_constant<int, 3>{}, sp + 3, s_alt, s_cur, ids[6], ids[7]);
                ids = nxt;
            }
        }
    }
    // the general steps: the rest in pairs (the two score sets alternate),
    // then the last one
    if (sp + kRing - 1 < steps) step_ids(sp + kRing - 1, nia, nib);
    for (; sp + 2 < steps; sp += 2) {
        step(std::false_type{}, General{}, sp, s_cur, s_alt, 0, 0);
        step(std::false_type{}, General{}, sp + 1, s_alt, s_cur, 0, 0);
    }
    if (sp + 1 < steps) {
        step(std::false_type{}, General{}, sp, s_cur, s_alt, 0, 0);
        step(std::true_type{}, General{}, sp + 1, s_alt, s_cur, 0, 0);
    } else if (sp < steps) {
        step(std::true_type{}, General{}, sp, s_cur, s_alt, 0, 0);
    }

    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));  // no load into LDS outlives the workgroup
    if constexpr (kDirectV) {
        // output elements 4 g4 .. + 3 with 4 g4 >= 8 (columns t >= 8 of the
        // V operands) were accumulated with each pair of operands swapped
        const bool sw = g4 >= 2;
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
            for (int i = 0; i < NV / 2; ++i) {
                const f32x4_t a = o[rb][2 * i], b = o[rb][2 * i + 1];
                o[rb][2 * i] = sw ? b : a;
                o[rb][2 * i + 1] = sw ? a : b;
            }
    }

    // ---- lane (t, g4) holds elements 16 j + 4 g4 .. + 3 of row t ----
    const float nan = __builtin_nanf("");
    constexpr int SLOT = prefix_slot_floats(D);
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
        const int r0 = row_w + rb * 16;
        if (r0 >= nrows) continue;  // wave-uniform
        float lt = l_run[rb] + lane_fetch(x16, l_run[rb]);
        lt += lane_fetch(x32, lt);  // weight sum of row t (over this chunk of keys)
        const int row = r0 + t;
        const size_t orow = (size_t)(q0 + min(row, nrows - 1) / G) * Hq + g * G + min(row, nrows - 1) % G;
        if (pf_chunks > 1 || (PFX && p.all_slots)) {
            // one chunk of several (or a prefix pass running beside the
            // suffix pass): the partial goes to its 16-row slot and the
            // merge launch that follows combines the chunks
            const int64_t f = pf_task16 + (int64_t)(r0 / 16) * (H * pf_chunks) + g * pf_chunks + pf_chunk;
            float* slotp = p.slots + (size_t)f * SLOT;
#pragma unroll
            for (int j = 0; j < NV; ++j)
                *reinterpret_cast<f32x4_t*>(slotp + t * D + 16 * j + 4 * g4) = o[rb][j];
            if (g4 == 0) {
                slotp[16 * D + t] = bad ? nan : m_run[rb];
                slotp[16 * D + 16 + t] = lt;
            }
        } else if constexpr (PFX) {
            // the prefix pass in one chunk: merge with the suffix results
            if (row < nrows) {
                const float m = bad ? nan : m_run[rb];
                const float lse = p.res_lse[orow];
                const float M = fmaxf(m, lse);
                const float wp = __builtin_amdgcn_exp2f(m - M);
                const float ws = __builtin_amdgcn_exp2f(lse - M);
                const float sc = p.v_scale / (wp * lt + ws);
#pragma unroll
                for (int j = 0; j < NV; ++j) {
                    const f32x4_t so = *reinterpret_cast<const f32x4_t*>(p.res_o + orow * D + 16 * j + 4 * g4);
                    store4_as<QT>(p.out, orow * D + 16 * j + 4 * g4, (wp * o[rb][j][0] + ws * so[0]) * sc,
                                  (wp * o[rb][j][1] + ws * so[1]) * sc, (wp * o[rb][j][2] + ws * so[2]) * sc,
                                  (wp * o[rb][j][3] + ws * so[3]) * sc);
                }
            }
        } else {
            // prefill in one chunk: normalise and store
            if (row < nrows) {
                const float sc = bad ? nan : p.v_scale / lt;
#pragma unroll
                for (int j = 0; j < NV; ++j)
                    store4_as<QT>(p.out, orow * D + 16 * j + 4 * g4, o[rb][j][0] * sc, o[rb][j][1] * sc,
                                  o[rb][j][2] * sc, o[rb][j][3] * sc);
            }
        }
    }
}

// The merge launch: one workgroup of 256 threads per (16-row block, KV head)
// of the rows whose keys were split into chunks (prefix groups in the prefix
// pass, PFX; prefill sequences with few rows otherwise). Thread i takes row
// i / 16 of the block and elements (i % 16) * D / 16 .. of it. With the
// block's slots f0 .. f0 + C - 1 (as the attention kernel placed them) and,
// in the prefix pass, the suffix result (o_s, lse_s) of the row (else
// lse_s = -inf):
//   M = max(m_1..m_C, lse_s),
//   out = v_scale * (sum_c 2^(m_c - M) acc_c + 2^(lse_s - M) o_s)
//                  / (sum_c 2^(m_c - M) l_c + 2^(lse_s - M)).
constexpr int kMergeThreads = 256;

template <int QT, int D, bool PFX>
__global__ __launch_bounds__(kMergeThreads) void chunk_merge_kernel(PrefillParams p) {
    constexpr int SLOT = prefix_slot_floats(D);
    constexpr int EPT = D / 16;  // elements per thread: 8 (d 128) or 4 (d 64)
    const int lane = lane_id();
    const int S = p.num_seqs, H = p.num_kv_heads, G = p.group, Hq = p.num_q_heads;
    // the units whose rows are stacked: prefix groups or prefill sequences
    int nu = S;
    if constexpr (PFX) {
        nu = usable_groups(p.group_starts, p.group_prefix, p.num_groups, S, p.max_blocks_per_seq, lane);
        if (nu == 0) return;
    }
    // unit j: its rows, row tiles, 16-row blocks and most chunks
    auto shape = [&](int j, int& rows, int& rts, int& rbs, int& cmax) {
        if constexpr (PFX) {
            const int pre = p.group_prefix[j];
            rows = pre > 0 ? (p.group_starts[j + 1] - p.group_starts[j]) * G : 0;
            rts = (rows + kGroupRows - 1) / kGroupRows;
            rbs = (rows + 15) / 16;
            cmax = pre;
        } else {
            int tmin = 0;
            prefill_seq_shape(p, j, rts, rbs, tmin);
            rows = rts > 0 ? (p.query_start[j + 1] - p.query_start[j]) * G : 0;
            cmax = max(tmin, 1);
        }
    };
    int rt_total = 0, rb_total = 0;
    for (int base = 0; base < nu; base += kWave) {
        const int j = base + lane;
        int rows = 0, rts = 0, rbs = 0, cmax = 0;
        if (j < nu) shape(j, rows, rts, rbs, cmax);
        rt_total += wave_sum_int(rts);
        rb_total += wave_sum_int(rbs);
    }
    if (rt_total == 0) return;
    const int cg = prefix_chunks(H, rt_total, rb_total, p.pf_target);
    const bool all_slots = PFX && p.all_slots;  // every group left slots
    if (cg == 1 && !all_slots) return;  // nothing was split: the attention kernel wrote every row
    const int g = blockIdx.x % H;
    const int rbg = blockIdx.x / H;  // 16-row block over all units
    if (rbg >= rb_total) return;
    // the block's unit (every wave finds the same)
    int rb_before = 0, jj = -1, rb16 = 0, C = 1, nrows = 0;
    int64_t t16_before = 0, t16 = 0;
    for (int base = 0; base < nu && jj < 0; base += kWave) {
        const int j = base + lane;
        int rows = 0, rts = 0, rbs = 0, cmax = 0;
        if (j < nu) shape(j, rows, rts, rbs, cmax);
        const int cj = min(cmax, cg);
        const int rincl = wave_inclusive_scan(rbs);
        const int tincl = wave_inclusive_scan(H * rbs * cj);
        const unsigned long long hit =
            __ballot(rbs > 0 && rb_before + rincl - rbs <= rbg && rbg < rb_before + rincl);
        if (hit) {
            const int L = __ffsll(hit) - 1;
            jj = base + L;
            rb16 = rbg - rb_before - __builtin_amdgcn_readlane(rincl - rbs, L);
            t16 = t16_before + __builtin_amdgcn_readlane(tincl - H * rbs * cj, L);
            C = __builtin_amdgcn_readlane(cj, L);
            nrows = __builtin_amdgcn_readlane(rows, L);
        }
        rb_before += __builtin_amdgcn_readlane(rincl, kWave - 1);
        t16_before += __builtin_amdgcn_readlane(tincl, kWave - 1);
    }
    if (jj < 0) return;  // not reached for rbg < rb_total
    if (C <= 1 && !all_slots) return;  // merged by the attention kernel
    const int r = threadIdx.x >> 4, e0 = (threadIdx.x & 15) * EPT;
    const int row = rb16 * 16 + r;
    if (row >= nrows) return;
    const int start = PFX ? p.group_starts[jj] : p.query_start[jj];  // a row's token = start + row / G
    const size_t orow = (size_t)(start + row / G) * Hq + g * G + row % G;
    const float* slot0 = p.slots + (size_t)(t16 + (int64_t)rb16 * (H * C) + g * C) * SLOT;
    const float lse = PFX ? p.res_lse[orow] : -INFINITY;
    float acc[EPT];
    f32x4_t so[EPT / 4];
#pragma unroll
    for (int i = 0; i < EPT; i += 4) {
        so[i / 4] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (PFX) so[i / 4] = *reinterpret_cast<const f32x4_t*>(p.res_o + orow * D + e0 + i);
    }
    constexpr int kPre = 8;
    if (C <= kPre) {
        // Every load of up to kPre chunks in one memory round (past the
        // last chunk: the last again, with weight zero), then the maximum,
        // the weights and the sums in chunk order.
        float mc[kPre], lc[kPre];
        f32x4_t ac[kPre][EPT / 4];
#pragma unroll
        for (int cc = 0; cc < kPre; ++cc) {
            const float* sl = slot0 + (size_t)min(cc, C - 1) * SLOT;
            mc[cc] = sl[16 * D + r];
            lc[cc] = sl[16 * D + 16 + r];
#pragma unroll
            for (int i = 0; i < EPT; i += 4) ac[cc][i / 4] = *reinterpret_cast<const f32x4_t*>(sl + r * D + e0 + i);
        }
        float M = lse;
#pragma unroll
        for (int cc = 0; cc < kPre; ++cc)
            if (cc < C) M = fmaxf(M, mc[cc]);
        const float ws = PFX ? __builtin_amdgcn_exp2f(lse - M) : 0.f;
        float L = ws;
#pragma unroll
        for (int i = 0; i < EPT; ++i) acc[i] = ws * so[i / 4][i % 4];
#pragma unroll
        for (int cc = 0; cc < kPre; ++cc) {
            // a chunk where the row saw no key holds m = -inf, l = 0 and zeros
            const float w = cc >= C || mc[cc] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc[cc] - M);
            L += w * lc[cc];
#pragma unroll
            for (int i = 0; i < EPT; ++i) acc[i] = fmaf(w, ac[cc][i / 4][i % 4], acc[i]);
        }
        const float sc = p.v_scale / L;
#pragma unroll
        for (int i = 0; i < EPT; i += 4)
            store4_as<QT>(p.out, orow * D + e0 + i, acc[i] * sc, acc[i + 1] * sc, acc[i + 2] * sc,
                          acc[i + 3] * sc);
        return;
    }
    float M = lse;
    // eight chunks' loads in flight at a time (a loop that is not unrolled
    // waits for each load before issuing the next)
#pragma unroll 8
    for (int cc = 0; cc < C; ++cc) M = fmaxf(M, slot0[(size_t)cc * SLOT + 16 * D + r]);
    const float ws = PFX ? __builtin_amdgcn_exp2f(lse - M) : 0.f;
    float L = ws;
#pragma unroll
    for (int i = 0; i < EPT; ++i) acc[i] = ws * so[i / 4][i % 4];
#pragma unroll 8
    for (int cc = 0; cc < C; ++cc) {
        const float* sl = slot0 + (size_t)cc * SLOT;
        // a chunk where the row saw no key holds m = -inf, l = 0 and zeros
        const float mc = sl[16 * D + r];
        const float w = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - M);
        L += w * sl[16 * D + 16 + r];
#pragma unroll
        for (int i = 0; i < EPT; i += 4) {
            const f32x4_t a = *reinterpret_cast<const f32x4_t*>(sl + r * D + e0 + i);
#pragma unroll
            for (int x = 0; x < 4; ++x) acc[i + x] = fmaf(w, a[x], acc[i + x]);
        }
    }
    const float sc = p.v_scale / L;
#pragma unroll
    for (int i = 0; i < EPT; i += 4)
        store4_as<QT>(p.out, orow * D + e0 + i, acc[i] * sc, acc[i + 1] * sc, acc[i + 2] * sc,
                      acc[i + 3] * sc);
}

// ---- dispatch ------------------------------------------------------------------

int64_t prefill_task_bound(int num_seqs, int num_tokens, int group, int num_kv_heads) {
    // sum over sequences of H * ceil(q_len * G / R) <= H * (T * G / R + S), R = kGroupRows
    return (int64_t)num_kv_heads * (((int64_t)num_tokens * group) / kGroupRows + num_seqs);
}

// Whether every (block, KV head) tile of a cache lies below 4 GiB from its
// start, so that the attention kernel may address tiles by 32-bit offsets.
template <int KT, int D>
static int tile_offsets_fit_32(int num_blocks, int num_kv_heads) {
    const uint64_t bytes = (uint64_t)num_blocks * (uint64_t)num_kv_heads * kBlock * D * Elem<KT>::bytes;
    return bytes <= 0xFFFFFFFFull ? 1 : 0;
}

template <int KT, int QT, int D>
static hipError_t launch_prefill_typed(const PrefillArgs& a) {
    PrefillParams p{};
    p.q = static_cast<const uint8_t*>(a.q);
    p.k_cache = static_cast<const uint8_t*>(a.k_cache);
    p.v_cache = static_cast<const uint8_t*>(a.v_cache);
    p.query_start = a.query_start;
    p.block_tables = a.block_tables;
    p.context_lens = a.context_lens;
    p.num_seqs = a.num_seqs;
    p.num_tokens = a.num_tokens;
    p.num_q_heads = a.num_q_heads;
    p.num_kv_heads = a.num_kv_heads;
    p.group = a.group;
    p.num_blocks = a.num_blocks;
    p.max_blocks_per_seq = a.max_blocks_per_seq;
    p.qk_scale_log2 = a.scale * (KT == PKV_FP8_E4M3 ? a.k_scale : 1.f) * 1.44269504088896340736f;
    p.v_scale = KT == PKV_FP8_E4M3 ? a.v_scale : 1.f;
    p.out = a.out;
    p.offsets32 = tile_offsets_fit_32<KT, D>(a.num_blocks, a.num_kv_heads);
    // The keys are split only when the row tiles (at least T * G / 128 per KV
    // head) fall short of the workgroup target; otherwise the workspace is
    // not touched and no merge launch is needed.
    const bool may_split = a.slots != nullptr &&
                           (int64_t)a.num_kv_heads * (((int64_t)a.num_tokens * a.group) / kGroupRows) <
                               kPrefixTargetWorkgroups;
    p.slots = may_split ? a.slots : nullptr;
    // with the key split: at most target + H * (row tiles) workgroups
    const int64_t grid = prefill_task_bound(a.num_seqs, a.num_tokens, a.group, a.num_kv_heads) +
                         (may_split ? kPrefixTargetWorkgroups : 0);
    if (grid <= 0) return hipSuccess;
    auto kernel = paged_prefill_kernel<KT, QT, D, false, 0>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kPrefillThreads), 0, a.stream, p, DecodeParams{}, 0);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || !may_split) return err;
    // the merge of split sequences (16-row blocks: at most T * G / 16 + S per KV head)
    const int64_t merge_grid = (int64_t)a.num_kv_heads *
                               (((int64_t)a.num_tokens * a.group) / 16 + a.num_seqs);
    auto merge = chunk_merge_kernel<QT, D, false>;
    hipLaunchKernelGGL(merge, dim3((unsigned)merge_grid), dim3(kMergeThreads), 0, a.stream, p);
    return hipGetLastError();
}

template <int KT, int QT>
static hipError_t launch_prefill_dim(const PrefillArgs& a) {
    return a.head_dim == 64 ? launch_prefill_typed<KT, QT, 64>(a) : launch_prefill_typed<KT, QT, 128>(a);
}

hipError_t launch_paged_prefill(const PrefillArgs& a) {
    if (a.kv_dtype == PKV_F32) return launch_prefill_dim<PKV_F32, PKV_F32>(a);
    if (a.kv_dtype == PKV_F16) return launch_prefill_dim<PKV_F16, PKV_F16>(a);
    if (a.kv_dtype == PKV_BF16) return launch_prefill_dim<PKV_BF16, PKV_BF16>(a);
    if (a.q_dtype == PKV_F16) return launch_prefill_dim<PKV_FP8_E4M3, PKV_F16>(a);
    return launch_prefill_dim<PKV_FP8_E4M3, PKV_BF16>(a);
}

// ---- the shared-prefix decode -------------------------------------------------
//
// Sequences that share a prefix reference one physical copy of its blocks
// (drpranayjha page, "How PagedAttention pages the KV cache"; ttlab page,
// section 4). Plain paged decode still reads such a block once per sequence.
// Here the suffix pass (the decode kernel in result mode, over each member's
// blocks after its group's prefix) leaves every member row's normalised
// output and log2-sum-exp in the workspace; the prefix pass is the kernel
// above in prefix mode: a group's (member, query head) rows are stacked like
// a prefill chunk's (token, head) rows, 128 to a workgroup, against the
// group's prefix blocks read once per workgroup through LDS. The prefix is
// split into chunks so that about kPrefixTargetWorkgroups workgroups run;
// chunk partials (16-row slots) are merged by a third launch, by the
// log-sum-exp rule, together with the suffix result.

// Beside the suffix pass, the prefix pass aims at fewer workgroups (its work
// hides under the suffix pass's stream, fewer of its workgroups take CUs from
// that stream, and fewer chunks leave fewer partials for the merge launch to
// read). 256 sequences sharing a 2048-token prefix, 32 / 8 heads: 106 us per
// call at a target of 64 (one chunk), 93 at 96 and 128 (two), 93.7 at 192,
// 96 at 256 and 106 at 384.
constexpr int kPrefixBesideTarget = 128;

// The prefix pass's parameters (beside: running beside the suffix pass).
template <int KT, int D>
static PrefillParams prefix_params(const DecodeArgs& a, bool beside) {
    PrefillParams p{};
    p.q = static_cast<const uint8_t*>(a.q);
    p.k_cache = static_cast<const uint8_t*>(a.k_cache);
    p.v_cache = static_cast<const uint8_t*>(a.v_cache);
    p.block_tables = a.block_tables;
    p.num_seqs = a.num_seqs;
    p.num_q_heads = a.num_q_heads;
    p.num_kv_heads = a.num_kv_heads;
    p.group = a.group;
    p.num_blocks = a.num_blocks;
    p.max_blocks_per_seq = a.max_blocks_per_seq;
    p.qk_scale_log2 = a.scale * (KT == PKV_FP8_E4M3 ? a.k_scale : 1.f) * 1.44269504088896340736f;
    p.v_scale = KT == PKV_FP8_E4M3 ? a.v_scale : 1.f;
    p.out = a.out;
    p.num_groups = a.num_groups;
    p.group_starts = a.group_starts;
    p.group_prefix = a.group_prefix;
    p.slots = a.prefix_slots;
    p.res_o = a.res_o;
    p.res_lse = a.res_lse;
    p.all_slots = beside ? 1 : 0;
    p.pf_target = beside ? kPrefixBesideTarget : kPrefixTargetWorkgroups;
    p.offsets32 = tile_offsets_fit_32<KT, D>(a.num_blocks, a.num_kv_heads);
    return p;
}

template <int KT, int QT, int D>
static hipError_t launch_prefix_typed(const DecodeArgs& a, bool beside, hipStream_t stream) {
    const PrefillParams p = prefix_params<KT, D>(a, beside);
    const int64_t grid = prefix_workgroup_bound(a.num_seqs, a.group, a.num_kv_heads, a.num_groups);
    auto kernel = paged_prefill_kernel<KT, QT, D, true, 0>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kPrefillThreads), 0, stream, p, DecodeParams{}, 0);
    return hipGetLastError();
}

// ---- the suffix and prefix passes in one launch (paged_prefill_kernel, FGM > 0) ----

template <int KT, int QT, int D, int GM>
static hipError_t launch_fused_typed(const DecodeArgs& a) {
    // the suffix pass's worker waves: as the decode launch would take them
    int nw = a.num_workers;
    if (nw == 0) {
        const int cus = device_cus();
        if (cus <= 0) return hipErrorInvalidDevice;
        nw = decode_waves_per_cu<KT, D, true>() * cus;
        if (nw > kMaxWorkers) nw = kMaxWorkers;
    }
    const int64_t unit_bound = (int64_t)a.num_seqs * a.num_kv_heads * a.max_blocks_per_seq;
    if (nw > unit_bound) nw = (int)unit_bound;
    if (nw < 1) nw = 1;
    const DecodeParams dp = decode_params<KT>(a, nw, 1, false, true);
    const PrefillParams pp = prefix_params<KT, D>(a, true);
    const int suffix_wgs = (nw + kPrefillWaves - 1) / kPrefillWaves;
    const int64_t grid =
        suffix_wgs + prefix_workgroup_bound(a.num_seqs, a.group, a.num_kv_heads, a.num_groups);
    hipLaunchKernelGGL((paged_prefill_kernel<KT, QT, D, true, GM>), dim3((unsigned)grid),
                       dim3(kPrefillThreads), 0, a.stream, pp, dp, suffix_wgs);
    return hipGetLastError();
}

template <int KT, int QT, int D>
static hipError_t launch_fused_group(const DecodeArgs& a) {
    switch (padded_group(a.group)) {
    case 1: return launch_fused_typed<KT, QT, D, 1>(a);
    case 2: return launch_fused_typed<KT, QT, D, 2>(a);
    case 4: return launch_fused_typed<KT, QT, D, 4>(a);
    case 6: return launch_fused_typed<KT, QT, D, 6>(a);
    default: return launch_fused_typed<KT, QT, D, 8>(a);
    }
}

template <int KT, int QT>
static hipError_t launch_fused_dim(const DecodeArgs& a) {
    return a.head_dim == 64 ? launch_fused_group<KT, QT, 64>(a) : launch_fused_group<KT, QT, 128>(a);
}

static hipError_t launch_fused(const DecodeArgs& a) {
    if (a.kv_dtype == PKV_F32) return launch_fused_dim<PKV_F32, PKV_F32>(a);
    if (a.kv_dtype == PKV_F16) return launch_fused_dim<PKV_F16, PKV_F16>(a);
    if (a.kv_dtype == PKV_BF16) return launch_fused_dim<PKV_BF16, PKV_BF16>(a);
    if (a.q_dtype == PKV_F16) return launch_fused_dim<PKV_FP8_E4M3, PKV_F16>(a);
    return launch_fused_dim<PKV_FP8_E4M3, PKV_BF16>(a);
}

template <int QT, int D>
static hipError_t launch_prefix_merge(const DecodeArgs& a, bool beside) {
    PrefillParams p{};
    p.num_seqs = a.num_seqs;
    p.num_q_heads = a.num_q_heads;
    p.num_kv_heads = a.num_kv_heads;
    p.group = a.group;
    p.max_blocks_per_seq = a.max_blocks_per_seq;
    p.v_scale = a.kv_dtype == PKV_FP8_E4M3 ? a.v_scale : 1.f;
    p.out = a.out;
    p.num_groups = a.num_groups;
    p.group_starts = a.group_starts;
    p.group_prefix = a.group_prefix;
    p.slots = a.prefix_slots;
    p.res_o = a.res_o;
    p.res_lse = a.res_lse;
    p.all_slots = beside ? 1 : 0;
    p.pf_target = beside ? kPrefixBesideTarget : kPrefixTargetWorkgroups;
    const int64_t merge_grid =
        (int64_t)a.num_kv_heads * prefix_row_blocks_bound(a.num_seqs, a.group, a.num_groups);
    auto merge = chunk_merge_kernel<QT, D, true>;
    hipLaunchKernelGGL(merge, dim3((unsigned)merge_grid), dim3(kMergeThreads), 0, a.stream, p);
    return hipGetLastError();
}

template <int KT, int QT>
static hipError_t launch_prefix_pass(const DecodeArgs& a, bool beside, hipStream_t stream) {
    return a.head_dim == 64 ? launch_prefix_typed<KT, QT, 64>(a, beside, stream)
                            : launch_prefix_typed<KT, QT, 128>(a, beside, stream);
}

static hipError_t prefix_pass(const DecodeArgs& a, bool beside, hipStream_t stream) {
    if (a.kv_dtype == PKV_F32) return launch_prefix_pass<PKV_F32, PKV_F32>(a, beside, stream);
    if (a.kv_dtype == PKV_F16) return launch_prefix_pass<PKV_F16, PKV_F16>(a, beside, stream);
    if (a.kv_dtype == PKV_BF16) return launch_prefix_pass<PKV_BF16, PKV_BF16>(a, beside, stream);
    if (a.q_dtype == PKV_F16) return launch_prefix_pass<PKV_FP8_E4M3, PKV_F16>(a, beside, stream);
    return launch_prefix_pass<PKV_FP8_E4M3, PKV_BF16>(a, beside, stream);
}

static hipError_t prefix_merge(const DecodeArgs& a, bool beside) {
    const int q = a.kv_dtype == PKV_FP8_E4M3 ? a.q_dtype : a.kv_dtype;
    const bool d64 = a.head_dim == 64;
    if (q == PKV_F32) return d64 ? launch_prefix_merge<PKV_F32, 64>(a, beside) : launch_prefix_merge<PKV_F32, 128>(a, beside);
    if (q == PKV_F16) return d64 ? launch_prefix_merge<PKV_F16, 64>(a, beside) : launch_prefix_merge<PKV_F16, 128>(a, beside);
    return d64 ? launch_prefix_merge<PKV_BF16, 64>(a, beside) : launch_prefix_merge<PKV_BF16, 128>(a, beside);
}

hipError_t launch_shared_prefix(const DecodeArgs& a) {
    // The prefix pass can run beside the suffix pass when it needs none of
    // the suffix results, i.e. when every 16-row block of every group can
    // leave its partial in a slot for the merge launch: then both passes are
    // one launch, and the merge follows.
    const bool fits = (int64_t)a.num_kv_heads *
                          prefix_row_blocks_bound(a.num_seqs, a.group, a.num_groups) <=
                      kPrefixSlots;
    if (fits) {
        hipError_t err = launch_fused(a);
        if (err == hipSuccess) err = prefix_merge(a, true);
        return err;
    }
    // otherwise one after the other: the suffix pass, then the prefix pass
    // (which merges one-chunk groups with the suffix results itself), then
    // the merge
    hipError_t err = launch_paged_decode(a);
    if (err == hipSuccess) err = prefix_pass(a, false, a.stream);
    if (err == hipSuccess) err = prefix_merge(a, false);
    return err;
}

}  // namespace pkv
