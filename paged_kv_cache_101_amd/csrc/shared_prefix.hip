// shared_prefix.hip -- the prefix pass of the shared-prefix decode.
//
// Sequences that share a prefix reference one physical copy of its blocks
// (drpranayjha page, "How PagedAttention pages the KV cache"; ttlab page,
// section 4). Plain paged decode still reads such a block once per sequence.
// Here each shared block is read once per KV head for 16 query rows at a
// time: the rows of a prefix group -- (member m, query head h of the KV head)
// -- are stacked 16 to an MFMA column set, so one K/V tile feeds 16
// (sequence, head) rows where decode feeds the G heads of one sequence. The
// per-tile arithmetic is decode's (TileMath): scores and P.V on the matrix
// cores, online softmax in log2 units.
//
// Tasks are (group, KV head g, row block of 16, chunk of the prefix blocks).
// The chunk count is the same for every group (capped by the group's prefix
// length), chosen so that the tasks number about target_tasks. A task's
// partial is its 16 rows' running max m, weight sum l and unnormalised
// accumulator. With one chunk the task merges it at once; otherwise it parks
// the partial in the workspace and the last of the row block's chunk tasks
// to finish (device-scope counter) merges them all. The merge also takes the
// suffix pass's result for each row (the normalised output of the blocks
// after the prefix and its log2-sum-exp, written by the decode kernel's
// suffix pass before this launch) and writes the output rows:
//   M = max(m_1..m_C, lse_s),
//   out = v_scale * (sum_c 2^(m_c - M) acc_c + 2^(lse_s - M) o_s)
//                  / (sum_c 2^(m_c - M) l_c + 2^(lse_s - M)).
#include "pkv_internal.h"
#include "pkv_tile.h"

namespace pkv {

namespace {

constexpr int kRows = 16;  // query rows per task: the MFMA column count

// Tiles a wave has in flight: up to 4, as many as 128 registers per lane
// hold (float32 tiles of 128 elements: 2).
constexpr int prefix_prefetch(int tile_dwords_per_lane) {
    return 128 / tile_dwords_per_lane >= 4 ? 4 : 128 / tile_dwords_per_lane < 1 ? 1 : 128 / tile_dwords_per_lane;
}

struct PrefixParams {
    const uint8_t* q;
    const uint8_t* k_cache;
    const uint8_t* v_cache;
    const int32_t* block_tables;
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int group;
    int num_blocks;
    int max_blocks_per_seq;
    int num_groups;
    const int32_t* group_starts;
    const int32_t* group_prefix;
    int target_tasks;
    float qk_scale_log2;
    float v_scale;
    int* counters;       // [H][row blocks], zero on entry and on exit
    float* slots;        // [tasks][prefix_slot_floats(D)] (used when chunks > 1)
    const float* res_o;  // suffix results [S][H_q][D]
    const float* res_lse;
    void* out;
};

// Where a task sits: its group's members [start, start + members) with
// `pre` shared blocks, chunk count C, and the counts of tasks and row blocks
// of the groups before it.
struct TaskGroup {
    int start, members, pre, rbs, chunks;
    int64_t task_base;
    int rb_base;
};

}  // namespace

template <int KT, int QT, int D>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(2)))
void shared_prefix_kernel(PrefixParams p) {
    using TM = TileMath<KT, QT, D>;
    constexpr int NK = TM::NK, NV = TM::NV, NVL = TM::NVL, KW = TM::KW, VLW = TM::VLW;
    constexpr int KB = Elem<KT>::bytes;
    constexpr int QB = Elem<QT>::bytes;
    constexpr uint32_t kTileBytes = (uint32_t)kBlock * D * KB;
    constexpr int SLOT = prefix_slot_floats(D);
    static_assert(D % kWave == 0, "head size must be a multiple of the wave width");

    const int lane = lane_id();
    const int S = p.num_seqs, H = p.num_kv_heads, G = p.group, Hq = p.num_q_heads;
    const int mb = p.max_blocks_per_seq;
    const float nan = __builtin_nanf("");
    const int ng = usable_groups(p.group_starts, p.group_prefix, p.num_groups, S, mb, lane);
    if (ng == 0) return;

    auto rows_of = [&](int j, int& start, int& members, int& pre) {
        start = p.group_starts[j];
        members = p.group_starts[j + 1] - start;
        pre = p.group_prefix[j];
    };
    auto rbs_of = [&](int members, int pre) { return pre > 0 ? (members * G + kRows - 1) / kRows : 0; };

    // Row blocks over all groups, the common chunk count, and the task count.
    int rb_total = 0;
    for (int base = 0; base < ng; base += kWave) {
        const int j = base + lane;
        int st = 0, m = 0, pre = 0;
        if (j < ng) rows_of(j, st, m, pre);
        rb_total += wave_sum_int(j < ng ? rbs_of(m, pre) : 0);
    }
    if (rb_total == 0) return;
    const int per_chunk = H * rb_total;  // tasks per chunk of every prefix
    const int cg = per_chunk >= p.target_tasks ? 1 : (p.target_tasks + per_chunk - 1) / per_chunk;
    int64_t total = 0;
    for (int base = 0; base < ng; base += kWave) {
        const int j = base + lane;
        int st = 0, m = 0, pre = 0;
        if (j < ng) rows_of(j, st, m, pre);
        total += wave_sum_int(j < ng ? H * rbs_of(m, pre) * min(pre, cg) : 0);
    }

    // The group holding task f (wave-uniform result).
    auto locate = [&](int64_t f) -> TaskGroup {
        TaskGroup tg{};
        int64_t tasks_before = 0;
        int rbs_before = 0;
        for (int base = 0; base < ng; base += kWave) {
            const int j = base + lane;
            int st = 0, m = 0, pre = 0;
            if (j < ng) rows_of(j, st, m, pre);
            const int rbs = j < ng ? rbs_of(m, pre) : 0;
            const int t = H * rbs * min(pre, cg);
            const int incl = wave_inclusive_scan(t, lane);
            const int rincl = wave_inclusive_scan(rbs, lane);
            const unsigned long long hit =
                __ballot(t > 0 && tasks_before + incl - t <= f && f < tasks_before + incl);
            if (hit) {
                const int L = __ffsll(hit) - 1;
                tg.start = __builtin_amdgcn_readlane(st, L);
                tg.members = __builtin_amdgcn_readlane(m, L);
                tg.pre = __builtin_amdgcn_readlane(pre, L);
                tg.rbs = __builtin_amdgcn_readlane(rbs, L);
                tg.chunks = min(tg.pre, cg);
                tg.task_base = tasks_before + __builtin_amdgcn_readlane(incl - t, L);
                tg.rb_base = rbs_before + __builtin_amdgcn_readlane(rincl - rbs, L);
                return tg;
            }
            tasks_before += __builtin_amdgcn_readlane(incl, kWave - 1);
            rbs_before += __builtin_amdgcn_readlane(rincl, kWave - 1);
        }
        return tg;  // not reached for f < total
    };

    // Lane roles, as in decode: column t = l % 16 (the query row for scores,
    // the token for K operands, the element for V operands and outputs) and
    // k-group g4 = l / 16.
    const int t = lane & 15;
    const int g4 = lane >> 4;
    const uint32_t k_off = (uint32_t)((g4 * kBlock + t) * 8 * KB);
    const uint32_t v_off = (uint32_t)((t * 4 + g4) * 8 * KB);
    const int x16 = (lane ^ 16) << 2, x32 = (lane ^ 32) << 2;
    int head_lane[4];  // lane holding row 4*g4 + r
#pragma unroll
    for (int j = 0; j < 4; ++j) head_lane[j] = (4 * g4 + j) << 2;
    const float qk_scale = p.qk_scale_log2;

    for (int64_t f = blockIdx.x; f < total; f += gridDim.x) {
        const TaskGroup tg = locate(f);
        const int C = tg.chunks;
        const int64_t i = f - tg.task_base;
        const int hc = H * C;
        const int rb = (int)(i / hc);
        const int g = (int)((i % hc) / C);
        const int c = (int)(i % C);
        const int nrows = tg.members * G;
        const int b0 = (int)((int64_t)c * tg.pre / C);
        const int b1 = (int)((int64_t)(c + 1) * tg.pre / C);
        const size_t bt_row = (size_t)tg.start * mb;  // the group's first member's table

        // this lane's query row (rows past the group's are zero and never stored)
        const int my_row = rb * kRows + t;
        const bool row_ok = my_row < nrows;
        const int s_row = tg.start + (row_ok ? my_row / G : 0);
        const int h_row = g * G + (row_ok ? my_row % G : 0);
        typename TM::Q q;
        TM::load_q(q, p.q + ((size_t)s_row * Hq + h_row) * D * QB, row_ok, g4);

        struct TileRef {
            size_t off;
            uint32_t bytes;
            bool bad;
        };
        auto tile_at = [&](int b) -> TileRef {
            if (b >= b1) return TileRef{0, 0u, false};
            const int id = uniform_read(p.block_tables, bt_row + b);
            if (id < 0 || id >= p.num_blocks) return TileRef{0, 0u, true};
            return TileRef{tile_elem_offset(id, g, H, D) * KB, kTileBytes, false};
        };
        // A ring of PF tiles in flight: tile b + PF is requested into the slot
        // that tile b leaves, K as soon as the scores are out, V after P.V.
        constexpr int PF = prefix_prefetch(NK * KW + NVL * VLW);
        uint32_t kr[PF][NK][KW], vr[PF][NVL][VLW];
        auto issue_k = [&](int slot, TileRef tr) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(p.k_cache + tr.off, tr.bytes);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < NK; ++k)
                load_dwords<KW, kLoadCached>(r, k_off + k * 4 * kBlock * 8 * KB, kr[slot][k]);
            __builtin_amdgcn_sched_barrier(0);
        };
        auto issue_v = [&](int slot, TileRef tr) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(p.v_cache + tr.off, tr.bytes);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < NVL; ++k)
                load_dwords<VLW, kLoadCached>(r, v_off + k * 32 * kBlock * KB, vr[slot][k]);
            __builtin_amdgcn_sched_barrier(0);
        };

        bool bad = false;
#pragma unroll
        for (int slot = 0; slot < PF; ++slot) {
            const TileRef tr = tile_at(b0 + slot);
            bad |= tr.bad;
            issue_k(slot, tr);
            issue_v(slot, tr);
        }
        float m_run = -INFINITY, l_run = 0.f;
        f32x4_t o[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // Every prefix block is full: no position is masked. A pass covers PF
        // tiles; slots past the chunk's last tile hold zeros (a buffer load
        // of size 0) and their scores are set to -inf.
        for (int b = b0; b < b1; b += PF) {
#pragma unroll
            for (int slot = 0; slot < PF; ++slot) {
                const bool live = b + slot < b1;
                const TileRef nxt = tile_at(b + slot + PF);
                bad |= nxt.bad;
                f32x4_t sc = TM::qk(kr[slot], q);
                settle(sc);
                issue_k(slot, nxt);
                float x[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = live ? sc[j] * qk_scale : -INFINITY;
                const float xm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
                if (__any(xm > m_run + kLazyRescale)) {
                    float tm = fmaxf(xm, lane_fetch(x16, xm));
                    tm = fmaxf(tm, lane_fetch(x32, tm));
                    const float mn = fmaxf(m_run, tm);
                    const float cf = __builtin_amdgcn_exp2f(m_run - mn);
                    l_run *= cf;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float cr = lane_fetch(head_lane[r], cf);
#pragma unroll
                        for (int j = 0; j < NV; ++j) o[j][r] *= cr;
                    }
                    m_run = mn;
                }
                float pr[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) pr[j] = __builtin_amdgcn_exp2f(x[j] - m_run);
                l_run += TM::pv(pr, vr[slot], o);
#pragma unroll
                for (int j = 0; j < NV; ++j) settle(o[j]);
                issue_v(slot, nxt);
            }
        }
        float lt = l_run + lane_fetch(x16, l_run);
        lt += lane_fetch(x32, lt);  // weight sum of row t over the chunk
        if (bad) m_run = nan;

        if (C == 1) {
            // the only chunk: merge with the suffix results from registers
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int hh = 4 * g4 + r;
                const float m_h = lane_fetch(head_lane[r], m_run);
                const float l_h = lane_fetch(head_lane[r], lt);
                const int row = rb * kRows + hh;
                if (row < nrows) {
                    const size_t orow = (size_t)(tg.start + row / G) * Hq + g * G + row % G;
                    const float lse = p.res_lse[orow];
                    const float M = fmaxf(m_h, lse);
                    const float wp = __builtin_amdgcn_exp2f(m_h - M);
                    const float ws = __builtin_amdgcn_exp2f(lse - M);
                    const float sc = p.v_scale / (wp * l_h + ws);
#pragma unroll
                    for (int j = 0; j < NV; ++j) {
                        const int e = 16 * j + t;
                        const float v = (wp * o[j][r] + ws * p.res_o[orow * D + e]) * sc;
                        store_f32_as<QT>(p.out, orow * D + e, v);
                    }
                }
            }
            continue;
        }

        // ---- several chunks: park the partial, the last one merges ----
        float* slotp = p.slots + (size_t)f * SLOT;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int hh = 4 * g4 + r;
#pragma unroll
            for (int j = 0; j < NV; ++j) coherent_store(slotp + hh * D + 16 * j + t, o[j][r]);
        }
        if (lane < kRows) {
            coherent_store(slotp + kRows * D + lane, m_run);
            coherent_store(slotp + kRows * D + kRows + lane, lt);
        }
        __builtin_amdgcn_s_waitcnt(0);  // the partial has landed before it is announced
        int* counter = p.counters + (size_t)g * rb_total + tg.rb_base + rb;
        int old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __builtin_amdgcn_readfirstlane(old);
        if (old != C - 1) continue;

        // The chunk partials of (group, g, rb) are slots f0 + c', c' < C.
        const int64_t f0 = f - c;
        auto slot_of = [&](int cc) { return p.slots + (size_t)(f0 + cc) * SLOT; };
        // per-row weights: lane r < 16 handles row r
        const int prow = rb * kRows + lane;
        const bool prow_ok = lane < kRows && prow < nrows;
        const size_t porow = prow_ok ? (size_t)(tg.start + prow / G) * Hq + g * G + prow % G : 0;
        const float lse = prow_ok ? p.res_lse[porow] : -INFINITY;
        float mx = lse;
        for (int cc = 0; cc < C; ++cc)
            mx = fmaxf(mx, lane < kRows ? coherent_load(slot_of(cc) + kRows * D + lane) : -INFINITY);
        const float ws = lane < kRows ? __builtin_amdgcn_exp2f(lse - mx) : 0.f;
        float L = ws;
        constexpr int PER_LANE = kRows * D / kWave;
        float acc[PER_LANE];
#pragma unroll
        for (int k = 0; k < PER_LANE; ++k) acc[k] = 0.f;
        for (int cc = 0; cc < C; ++cc) {
            const float* sl = slot_of(cc);
            const float wc = lane < kRows ? __builtin_amdgcn_exp2f(coherent_load(sl + kRows * D + lane) - mx) : 0.f;
            L += lane < kRows ? wc * coherent_load(sl + kRows * D + kRows + lane) : 0.f;
#pragma unroll
            for (int k = 0; k < PER_LANE; ++k) {
                // element k * 64 + lane is row (k * 64) / D, known at compile time
                const float w = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wc), (k * kWave) / D));
                acc[k] = fmaf(w, coherent_load(sl + k * kWave + lane), acc[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < PER_LANE; ++k) {
            const int rr = (k * kWave) / D, e = (k * kWave + lane) % D;
            const int row = rb * kRows + rr;
            const float w_s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ws), rr));
            const float l_r = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, L), rr));
            if (row < nrows) {
                const size_t orow = (size_t)(tg.start + row / G) * Hq + g * G + row % G;
                const float v = (acc[k] + w_s * p.res_o[orow * D + e]) * (p.v_scale / l_r);
                store_f32_as<QT>(p.out, orow * D + e, v);
            }
        }
        if (lane == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---- dispatch ------------------------------------------------------------------

template <int KT, int QT, int D>
static hipError_t launch_prefix_typed(const DecodeArgs& a) {
    PrefixParams p;
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
    p.num_groups = a.num_groups;
    p.group_starts = a.group_starts;
    p.group_prefix = a.group_prefix;
    p.target_tasks = kPrefixTargetTasks;
    p.qk_scale_log2 = a.scale * (KT == PKV_FP8_E4M3 ? a.k_scale : 1.f) * 1.44269504088896340736f;
    p.v_scale = KT == PKV_FP8_E4M3 ? a.v_scale : 1.f;
    p.counters = a.prefix_counters;
    p.slots = a.prefix_slots;
    p.res_o = a.res_o;
    p.res_lse = a.res_lse;
    p.out = a.out;
    // At most max(H * row blocks, 2 * target) tasks exist (the chunk count is
    // 1 when the row blocks alone reach the target); waves stride over them.
    const int64_t bound = prefix_task_bound(a.num_seqs, a.group, a.num_kv_heads, a.num_groups);
    const int grid = (int)(bound < 2 * kPrefixTargetTasks ? bound : 2 * kPrefixTargetTasks);
    auto kernel = shared_prefix_kernel<KT, QT, D>;
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kWave), 0, a.stream, p);
    return hipGetLastError();
}

template <int KT, int QT>
static hipError_t launch_prefix_dim(const DecodeArgs& a) {
    return a.head_dim == 64 ? launch_prefix_typed<KT, QT, 64>(a) : launch_prefix_typed<KT, QT, 128>(a);
}

hipError_t launch_shared_prefix(const DecodeArgs& a) {
    // the suffix pass (decode kernel, result mode), then the prefix pass
    hipError_t err = launch_paged_decode(a);
    if (err != hipSuccess) return err;
    if (a.kv_dtype == PKV_F32) return launch_prefix_dim<PKV_F32, PKV_F32>(a);
    if (a.kv_dtype == PKV_F16) return launch_prefix_dim<PKV_F16, PKV_F16>(a);
    if (a.kv_dtype == PKV_BF16) return launch_prefix_dim<PKV_BF16, PKV_BF16>(a);
    if (a.q_dtype == PKV_F16) return launch_prefix_dim<PKV_FP8_E4M3, PKV_F16>(a);
    return launch_prefix_dim<PKV_FP8_E4M3, PKV_BF16>(a);
}

}  // namespace pkv
