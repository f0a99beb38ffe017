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
//   * The sequence's 16-token tiles stream through an LDS ring of three
//     two-tile steps, two steps ahead of the one computed, moved from L2
//     straight into LDS by direct loads (no registers). Each wave reads a
//     step's K and V operands from LDS once and applies them to its 32 rows:
//     a tile costs one L2 read per 128 rows. P.V contracts both tiles of a
//     step in one 16x16x32 MFMA per 16 output columns.
//   * Per 16-row block the arithmetic is decode's (TileMath): S^T = K . Q^T and
//     O += P . V on MFMA, online softmax in log2 units with a lazily moved
//     maximum. Tiles wholly before a row block's first position need no mask;
//     the diagonal tiles mask key k > p per row by select; tiles after its last
//     position are skipped.
//   * Workgroup index -> (sequence, row tile, KV head) with the KV head fastest,
//     so the workgroups of one head land on one XCD (workgroups are dealt to
//     the 8 XCDs round-robin) and share its L2; within a sequence the row
//     tiles with the most keys start first.
#include "pkv_internal.h"
#include "pkv_tile.h"

namespace pkv {

namespace {

constexpr int kPrefillWaves = 4;                    // waves per workgroup
constexpr int kRowBlocks = 2;                       // 16-row blocks per wave
constexpr int kWaveRows = 16 * kRowBlocks;          // 32
constexpr int kGroupRows = kPrefillWaves * kWaveRows;  // 128
constexpr int kPrefillThreads = kPrefillWaves * kWave;
constexpr int kRing = 3;  // LDS ring of two-tile steps: kRing - 1 steps in flight

// s_waitcnt operand that waits for the vector-memory counter to reach n
// (expcnt and lgkmcnt left at their maxima; gfx9 encoding, vmcnt split
// over bits 3:0 and 15:14).
constexpr int vmcnt_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// SZ bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds_base + l * SZ (lds_base is the same for the whole wave).
template <int SZ>
__device__ __forceinline__ void load_to_lds(const uint8_t* src, uint8_t* lds_base) {
    static_assert(SZ == 16, "load size");
    __builtin_amdgcn_global_load_lds((const void*)src,
                                     (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// Wait until at most n (0..8, wave-uniform) of this wave's vector-memory
// operations are in flight: s_waitcnt takes its count as an immediate.
__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_wait(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_wait(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_wait(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_wait(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_wait(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_wait(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(vmcnt_wait(6)); break;
    case 7: __builtin_amdgcn_s_waitcnt(vmcnt_wait(7)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_wait(8)); break;
    }
}

// All waves of the workgroup reach this point. A compiler barrier on both
// sides keeps memory accesses from moving across it; unlike __syncthreads()
// it does not wait for this wave's outstanding loads.
__device__ __forceinline__ void workgroup_barrier() {
    asm volatile("" ::: "memory");
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
};

// Row tiles of kGroupRows rows of a sequence (0 for an invalid chunk).
__device__ __forceinline__ int row_tiles(const PrefillParams& p, int s) {
    const int a = p.query_start[s], b = p.query_start[s + 1];
    const int n = p.context_lens[s];
    if (a < 0 || b < a || b > p.num_tokens || n > p.max_blocks_per_seq * kBlock || b - a > n)
        return 0;
    return ((b - a) * p.group + kGroupRows - 1) / kGroupRows;
}

}  // namespace

template <int KT, int QT, int D>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(2)))
void paged_prefill_kernel(PrefillParams p) {
    using TM = TileMath<KT, QT, D>;
    constexpr int NK = TM::NK, NV = TM::NV, NVL = TM::NVL, KW = TM::KW, VLW = TM::VLW;
    constexpr int KB = Elem<KT>::bytes;
    constexpr int QB = Elem<QT>::bytes;
    constexpr uint32_t kTileBytes = (uint32_t)kBlock * D * KB;

    // kRing stages of two tiles' (K, V)
    __shared__ __attribute__((aligned(16))) uint8_t lds[kRing * 4 * kTileBytes];

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
    const int rt = row_tiles(p, s) - 1 - local / H;  // the longest row tiles first
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

    // ---- the tile stream: an LDS ring of two-tile steps, filled by direct loads ----
    // A step is tiles 2 * sp (A) and 2 * sp + 1 (B); it goes to ring stage
    // sp % kRing, kRing - 1 steps ahead of the one computed. A step is moved
    // from L2 straight into LDS (no registers) in 1 KiB pieces, 16 bytes per
    // lane: piece c (A's K, A's V, B's K, B's V, in that order) is carried by
    // wave c % 8. A wave waits for its own loads of step sp (the counter counts
    // its loads in issue order), then the barrier makes every wave's pieces
    // visible; the stage refilled after that barrier was last read before it.
    // A tile B past the last one reads the null block (it is masked out), so
    // every step issues the same loads.
    constexpr int kPieces = 2 * (int)kTileBytes / 1024;  // of one tile: its K, then its V
    constexpr int kStepPieces = 2 * kPieces;
    constexpr uint32_t kStepBytes = 4 * kTileBytes;
    constexpr int kWavePieces = (kStepPieces + kPrefillWaves - 1) / kPrefillWaves;  // at most
    static_assert(kTileBytes % 1024 == 0 && kWavePieces <= 8, "piece split");
    const int my_pieces = (kStepPieces - wv + kPrefillWaves - 1) / kPrefillWaves;
    const int steps = (tiles + 1) / 2;
    // V pieces are stored permuted so that the V operand reads are
    // lane-contiguous (free of LDS bank conflicts): a lane's V load i is
    // kVChunks 16-byte chunks (tokens 4 * g4 .. + 3 of its element columns),
    // found at chunk 4 * t + g4 (times kVChunks) of their region of the tile;
    // the piece's lane L fetches the chunk that reading lane L needs. fp8 V
    // loads are 8 bytes per lane and are stored as they are.
    constexpr int kVChunks = VLW / 4;
    auto v_piece_src = [&](int pc) -> uint32_t {
        if constexpr (kVChunks > 0) {
            const int i = pc / kVChunks, h = pc % kVChunks;
            const int sigma = 4 * (lane & 15) + (lane >> 4);  // 4 * t + g4 of reading lane L
            return (uint32_t)(i * 1024 * kVChunks + (kVChunks * sigma + h) * 16);
        } else {
            return (uint32_t)pc * 1024 + (uint32_t)lane * 16;
        }
    };
    bool bad = false;
    auto issue = [&](int sp) {
        const uint32_t st = (uint32_t)(sp % kRing) * kStepBytes;
        size_t off[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int j = 2 * sp + h2;
            int id = 0;  // past the last tile: the null block, masked out
            if (j < tiles) {
                id = uniform_read(p.block_tables, bt_row + j);
                if (id < 0 || id >= p.num_blocks) {
                    bad = true;  // its rows become NaN; the null block is read instead
                    id = 0;
                }
            }
            off[h2] = tile_elem_offset(id, g, H, D) * KB;
        }
#pragma unroll
        for (int i = 0; i < kWavePieces; ++i) {
            const int c = wv + i * kPrefillWaves;
            if (c < kStepPieces) {
                const int th = c / kPieces;  // 0: tile A, 1: tile B
                const int cc = c % kPieces;
                const bool is_v = cc >= kPieces / 2;
                const int pc = is_v ? cc - kPieces / 2 : cc;
                const uint32_t src = is_v ? v_piece_src(pc) : (uint32_t)pc * 1024 + (uint32_t)lane * 16;
                load_to_lds<16>((is_v ? p.v_cache : p.k_cache) + off[th] + src,
                                lds + st + (uint32_t)th * 2 * kTileBytes + (is_v ? kTileBytes : 0) +
                                    (uint32_t)pc * 1024);
            }
        }
    };
    // wait until at most `later` steps' loads of this wave are in flight
    auto wait_steps = [&](int later) {
        static_assert(kRing == 3, "later is 0 or 1");
        wait_vmcnt(later > 0 ? my_pieces : 0);
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

    auto read_k = [&](uint32_t base, uint32_t (&kr)[NK][KW]) {
#pragma unroll
        for (int i = 0; i < NK; ++i)
#pragma unroll
            for (int c = 0; c < KW; ++c)
                kr[i][c] = reinterpret_cast<const uint32_t*>(lds + base + k_off + i * 4 * kBlock * 8 * KB)[c];
    };
    auto read_v = [&](uint32_t base, uint32_t (&vr)[NVL][VLW]) {
        if constexpr (kVChunks > 0) {
            // the permuted store: this lane's 16-byte chunks sit at lane * 16
#pragma unroll
            for (int i = 0; i < NVL; ++i)
#pragma unroll
                for (int h = 0; h < kVChunks; ++h)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        vr[i][4 * h + c] = reinterpret_cast<const uint32_t*>(
                            lds + base + (kVChunks * i + h) * 1024 + lane * 16)[c];
        } else {
#pragma unroll
            for (int i = 0; i < NVL; ++i)
#pragma unroll
                for (int c = 0; c < VLW; ++c)
                    vr[i][c] = reinterpret_cast<const uint32_t*>(lds + base + v_off + i * 32 * kBlock * KB)[c];
        }
    };

    for (int sp = 0; sp < kRing - 1 && sp < steps; ++sp) issue(sp);
    for (int sp = 0; sp < steps; ++sp) {
        const uint32_t st = (uint32_t)(sp % kRing) * kStepBytes;
        wait_steps(min(kRing - 2, steps - 1 - sp));
        workgroup_barrier();
        if (sp + kRing - 1 < steps) issue(sp + kRing - 1);
        const int key0 = 2 * sp * kBlock;  // first key of tile A; tile B starts at key0 + 16
        const bool has_b = 2 * sp + 1 < tiles;
        bool any = false;  // a row block of this wave sees a key of the step
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb) any |= rb_last[rb] >= key0;
        if (!any) continue;
        // scores of both tiles for every row block
        f32x4_t sa[kRowBlocks], sb[kRowBlocks];
        {
            uint32_t kr[NK][KW];
            read_k(st, kr);
#pragma unroll
            for (int rb = 0; rb < kRowBlocks; ++rb) sa[rb] = TM::qk(kr, q[rb]);
            read_k(st + 2 * kTileBytes, kr);
#pragma unroll
            for (int rb = 0; rb < kRowBlocks; ++rb) sb[rb] = TM::qk(kr, q[rb]);
        }
        uint32_t va[NVL][VLW], vb[NVL][VLW];
        read_v(st + kTileBytes, va);
        read_v(st + 3 * kTileBytes, vb);
        // Keys at or past n (the unused rows of the last block), and a tile B
        // past the workgroup's last tile (which the causal limit, not n, can
        // end), are seen by no row: their V elements are zeroed, so that
        // whatever those rows hold cannot reach P . V (their scores are
        // excluded by select below).
        if (key0 + kBlock > n) TM::mask_v(va, n - key0 - 4 * g4);
        if (!has_b) TM::mask_v(vb, 0);  // the null block stands in for a missing tile B
        else if (key0 + 2 * kBlock > n) TM::mask_v(vb, n - key0 - kBlock - 4 * g4);
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb) {
            if (rb_last[rb] < key0) continue;  // no row of the block sees this step
            float xa[4], xb[4];
            if (key0 + 2 * kBlock - 1 <= rb_first[rb]) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xa[e] = sa[rb][e] * qk_scale;
                    xb[e] = sb[rb][e] * qk_scale;
                }
            } else {
                // a diagonal step: key k of this lane is key0 + 4 * g4 + e (A)
                // and key0 + 16 + 4 * g4 + e (B)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xa[e] = key0 + 4 * g4 + e <= pos[rb] ? sa[rb][e] * qk_scale : -INFINITY;
                    xb[e] = has_b && key0 + kBlock + 4 * g4 + e <= pos[rb] ? sb[rb][e] * qk_scale
                                                                           : -INFINITY;
                }
            }
            const float xm = fmaxf(fmaxf(fmaxf(xa[0], xa[1]), fmaxf(xa[2], xa[3])),
                                   fmaxf(fmaxf(xb[0], xb[1]), fmaxf(xb[2], xb[3])));
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
            float pa[4], pb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pa[e] = __builtin_amdgcn_exp2f(xa[e] - m_run[rb]);
                pb[e] = __builtin_amdgcn_exp2f(xb[e] - m_run[rb]);
            }
            if constexpr (TM::kF32) {
                l_run[rb] += TM::pv(pa, va, o[rb]);
                l_run[rb] += TM::pv(pb, vb, o[rb]);
            } else {
                l_run[rb] += TM::pv2(pa, pb, va, vb, o[rb]);
            }
        }
    }

    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));  // no load into LDS outlives the workgroup

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
    // sum over sequences of H * ceil(q_len * G / R) <= H * (T * G / R + S), R = kGroupRows
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
