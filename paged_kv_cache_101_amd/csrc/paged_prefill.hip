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
//   * A workgroup of 4 waves owns 256 query rows of one (sequence, KV head),
//     stacked token-major (row = token * G + head), 64 per wave as four
//     16-row MFMA column sets.
//   * The sequence's 16-token tiles stream through LDS, double-buffered: the
//     workgroup loads tile j+1 from L2 (one 16-byte piece per thread for a
//     16-bit d 128 tile) while computing tile j. Each wave reads a tile's K
//     and V operands from LDS once and applies them to its 64 rows, so a tile
//     costs one L2 read per 256 rows and one LDS read per 64 rows.
//   * Per 16-row block the arithmetic is decode's (TileMath): S^T = K . Q^T and
//     O += P . V on MFMA, online softmax in log2 units with a lazily moved
//     maximum. Tiles wholly before a row block's first position need no mask;
//     the diagonal tiles mask key k > p per row by select; tiles after its last
//     position are skipped.
//   * Workgroup index -> (sequence, row tile, KV head) with the KV head fastest,
//     so the workgroups of one head land on one XCD (workgroups are dealt to
//     the 8 XCDs round-robin) and share its L2.
#include "pkv_internal.h"
#include "pkv_tile.h"

namespace pkv {

namespace {

constexpr int kPrefillWaves = 4;                    // waves per workgroup
constexpr int kRowBlocks = 4;                       // 16-row blocks per wave
constexpr int kWaveRows = 16 * kRowBlocks;          // 64
constexpr int kGroupRows = kPrefillWaves * kWaveRows;  // 256
constexpr int kPrefillThreads = kPrefillWaves * kWave;

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
};

// Row tiles of 256 rows of a sequence (0 for an invalid chunk).
__device__ __forceinline__ int row_tiles(const PrefillParams& p, int s) {
    const int a = p.query_start[s], b = p.query_start[s + 1];
    const int n = p.context_lens[s];
    if (a < 0 || b < a || b > p.num_tokens || n > p.max_blocks_per_seq * kBlock || b - a > n)
        return 0;
    return ((b - a) * p.group + kGroupRows - 1) / kGroupRows;
}

}  // namespace

template <int KT, int QT, int D>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(1)))
void paged_prefill_kernel(PrefillParams p) {
    using TM = TileMath<KT, QT, D>;
    constexpr int NK = TM::NK, NV = TM::NV, NVL = TM::NVL, KW = TM::KW, VLW = TM::VLW;
    constexpr int KB = Elem<KT>::bytes;
    constexpr int QB = Elem<QT>::bytes;
    constexpr uint32_t kTileBytes = (uint32_t)kBlock * D * KB;
    constexpr int kPieceDwords = kTileBytes / 4 / kPrefillThreads;  // per thread and cache
    static_assert(kPieceDwords >= 1 && kTileBytes % (4 * kPrefillThreads) == 0, "tile split");

    // two stages of (K tile, V tile)
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kTileBytes];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wv = wave_id();
    const int S = p.num_seqs, H = p.num_kv_heads, G = p.group, Hq = p.num_q_heads;

    // ---- this workgroup's (sequence, row tile, KV head) ----
    const int task = blockIdx.x;
    int s = -1, local = 0;
    {
        int before = 0;
        for (int base = 0; base < S; base += kWave) {
            const int ss = base + lane;
            const int c = ss < S ? row_tiles(p, ss) * H : 0;
            const int incl = wave_inclusive_scan(c, lane);
            const unsigned long long hit = __ballot(c > 0 && before + incl - c <= task &&
                                                    task < before + incl);
            if (hit) {
                const int L = __ffsll(hit) - 1;
                s = base + L;
                local = task - before - __builtin_amdgcn_readlane(incl - c, L);
                break;
            }
            before += __builtin_amdgcn_readlane(incl, kWave - 1);
        }
    }
    if (s < 0) return;  // the grid is an upper bound on the tasks
    const int g = local % H;
    const int rt = local / H;
    const int q0 = p.query_start[s];
    const int q_len = p.query_start[s + 1] - q0;
    const int n = p.context_lens[s];
    const int nrows = q_len * G;
    const int base_pos = n - q_len;  // position of the chunk's first token
    const int row_wg = rt * kGroupRows;
    const int last_row = min(nrows, row_wg + kGroupRows) - 1;
    const int tiles = (base_pos + last_row / G) / kBlock + 1;  // keys 0 .. last position
    const size_t bt_row = (size_t)s * p.max_blocks_per_seq;

    // ---- per lane: its query row in each of the wave's four row blocks ----
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
        pos[rb] = base_pos + tok;
        const int h = g * G + (ok ? row % G : 0);
        TM::load_q(q[rb], p.q + ((size_t)(q0 + tok) * Hq + h) * D * QB, ok, g4);
    }
    // row-block extents (wave-uniform): first and last valid position
    int rb_first[kRowBlocks], rb_last[kRowBlocks];
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
        const int r0 = row_w + rb * 16;
        const int r1 = min(nrows, r0 + 16) - 1;
        rb_first[rb] = r0 < nrows ? base_pos + r0 / G : INT32_MAX;
        rb_last[rb] = r0 < nrows ? base_pos + r1 / G : -1;
    }

    // ---- the tile stream through LDS ----
    bool bad = false;
    auto tile_ref = [&](int j, uint32_t& bytes) -> size_t {
        bytes = 0;
        if (j >= tiles) return 0;
        const int id = uniform_read(p.block_tables, bt_row + j);
        if (id < 0 || id >= p.num_blocks) {
            bad = true;
            return 0;
        }
        bytes = kTileBytes;
        return tile_elem_offset(id, g, H, D) * KB;
    };
    uint32_t sk[kPieceDwords], sv[kPieceDwords];
    const uint32_t piece = (uint32_t)tid * kPieceDwords * 4;
    auto fetch = [&](int j) {
        uint32_t bytes;
        const size_t off = tile_ref(j, bytes);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_cache + off, bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_cache + off, bytes);
        load_dwords<kPieceDwords, kLoadCached>(rk, piece, sk);
        load_dwords<kPieceDwords, kLoadCached>(rv, piece, sv);
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kPieceDwords; ++i) {
            reinterpret_cast<uint32_t*>(lds[buf][0] + piece)[i] = sk[i];
            reinterpret_cast<uint32_t*>(lds[buf][1] + piece)[i] = sv[i];
        }
    };

    const uint32_t k_off = (uint32_t)((g4 * kBlock + t) * 8 * KB);
    const uint32_t v_off = (uint32_t)((t * 4 + g4) * 8 * KB);
    const int x16 = (lane ^ 16) << 2, x32 = (lane ^ 32) << 2;
    int head_lane[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) head_lane[j] = (4 * g4 + j) << 2;
    const float qk_scale = p.qk_scale_log2;

    float m_run[kRowBlocks], l_run[kRowBlocks];
    f32x4_t o[kRowBlocks][NV];
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) o[rb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    fetch(0);
    stage(0);
    __syncthreads();
    for (int j = 0; j < tiles; ++j) {
        const int buf = j & 1;
        fetch(j + 1);  // in flight while tile j is computed
        const int key0 = j * kBlock;
        // the wave's row blocks that see any key of tile j
        bool any = false;
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb) any |= rb_last[rb] >= key0;
        if (any) {
            uint32_t kr[NK][KW], vr[NVL][VLW];
#pragma unroll
            for (int i = 0; i < NK; ++i)
#pragma unroll
                for (int c = 0; c < KW; ++c)
                    kr[i][c] = reinterpret_cast<const uint32_t*>(
                        lds[buf][0] + k_off + i * 4 * kBlock * 8 * KB)[c];
#pragma unroll
            for (int i = 0; i < NVL; ++i)
#pragma unroll
                for (int c = 0; c < VLW; ++c)
                    vr[i][c] = reinterpret_cast<const uint32_t*>(
                        lds[buf][1] + v_off + i * 32 * kBlock * KB)[c];
            // Keys at or past n (the unused rows of the last block) are seen by
            // no row: their V elements are zeroed, so that whatever those rows
            // hold cannot reach P . V (their scores are excluded by select).
            if (key0 + kBlock > n) TM::mask_v(vr, n - key0 - 4 * g4);
#pragma unroll
            for (int rb = 0; rb < kRowBlocks; ++rb) {
                if (rb_last[rb] < key0) continue;  // no row of the block sees tile j
                const f32x4_t sc = TM::qk(kr, q[rb]);
                float x[4];
                if (key0 + kBlock - 1 <= rb_first[rb]) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = sc[e] * qk_scale;
                } else {
                    // diagonal tile: key k of this lane is key0 + 4 * g4 + e
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        x[e] = key0 + 4 * g4 + e <= pos[rb] ? sc[e] * qk_scale : -INFINITY;
                }
                const float xm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
                if (__any(xm > m_run[rb] + kLazyRescale)) {
                    float tm = fmaxf(xm, lane_fetch(x16, xm));
                    tm = fmaxf(tm, lane_fetch(x32, tm));
                    const float mn = fmaxf(m_run[rb], tm);
                    const float cf = __builtin_amdgcn_exp2f(m_run[rb] - mn);
                    l_run[rb] *= cf;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float cr = lane_fetch(head_lane[r], cf);
#pragma unroll
                        for (int e = 0; e < NV; ++e) o[rb][e][r] *= cr;
                    }
                    m_run[rb] = mn;
                }
                float pr[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) pr[e] = __builtin_amdgcn_exp2f(x[e] - m_run[rb]);
                l_run[rb] += TM::pv(pr, vr, o[rb]);
            }
        }
        if (j + 1 < tiles) {
            stage(buf ^ 1);  // the other buffer was last read before the previous barrier
        }
        __syncthreads();
    }

    // ---- normalise and store the wave's rows ----
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
        float lt = l_run[rb] + lane_fetch(x16, l_run[rb]);
        lt += lane_fetch(x32, lt);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float sc = p.v_scale / lane_fetch(head_lane[r], lt);
            const int row = row_w + rb * 16 + 4 * g4 + r;
            if (row < nrows) {
                const size_t orow = (size_t)(q0 + row / G) * Hq + g * G + row % G;
#pragma unroll
                for (int e = 0; e < NV; ++e)
                    store_f32_as<QT>(p.out, orow * D + 16 * e + t, bad ? nan : o[rb][e][r] * sc);
            }
        }
    }
}

// ---- dispatch ------------------------------------------------------------------

int64_t prefill_task_bound(int num_seqs, int num_tokens, int group, int num_kv_heads) {
    // sum over sequences of H * ceil(q_len * G / 256) <= H * (T * G / 256 + S)
    return (int64_t)num_kv_heads * (((int64_t)num_tokens * group) / kGroupRows + num_seqs);
}

template <int KT, int QT, int D>
static hipError_t launch_prefill_typed(const PrefillArgs& a) {
    PrefillParams p;
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
    const int64_t grid = prefill_task_bound(a.num_seqs, a.num_tokens, a.group, a.num_kv_heads);
    if (grid <= 0) return hipSuccess;
    auto kernel = paged_prefill_kernel<KT, QT, D>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kPrefillThreads), 0, a.stream, p);
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

}  // namespace pkv
