// paged_decode.hip -- paged decode attention for gfx950 (CDNA4), one launch.
//
// What is computed (ttlab page, sections 2 and 4; drpranayjha page, "How
// PagedAttention pages the KV cache"; tarundecipher page, "Batching does not
// merge the conversations"): one query token per sequence attends over the
// sequence's own K/V rows, found through its block table in a shared pool of
// 16-token physical blocks; a group of G query heads shares one KV head.
//
// Work decomposition: a persistent, evenly split tile stream
//   * A "tile" is one (sequence s, KV head g, logical block b): 16 K rows and
//     16 V rows of D elements, contiguous in the pool. All tiles of the batch
//     are numbered s-major, then g, then b. Each worker wave takes an equal
//     contiguous slice of that numbering (within one tile of every other
//     wave), whatever the mix of sequence lengths.
//   * A wave streams its slice: the K and V tiles of the next tile are in
//     flight while the current one is computed (K of the next is issued as
//     soon as the current QK is done, V after the current P.V).
//   * A slice covers whole (s, g) segments and at most two partial ones. A
//     segment finished by one wave is written out directly. A segment split
//     over several waves (the split-KV case) leaves one partial (running max
//     m, sum l, unnormalised accumulator) per wave in the workspace; the last
//     wave to finish the segment, found with a device-scope counter, merges
//     them with the log-sum-exp rule and writes the output.
//   * Tiles are 16 rows x D elements. A lane owns 8 consecutive elements of a
//     row, so D/8 lanes cover a row and one wave instruction covers 64*8
//     contiguous elements: every load is coalesced and goes straight to
//     registers; cache tiles use nontemporal loads (read once).
//   * QK: per-lane dot products (dot2 instructions for 16-bit data), then a
//     DPP sum across the D/8 lanes of the row. Online softmax in log2 units
//     with a lazily moved maximum; P.V accumulates in float32.
// Positions >= n inside a sequence's last block are excluded by select
// (score -inf, V row zero), never by arithmetic, so garbage or NaN there
// cannot leak.
#include <atomic>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

struct DecodeParams {
    const uint8_t* q;
    const uint8_t* k_cache;
    const uint8_t* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int group;
    int num_blocks;
    int max_blocks_per_seq;
    int num_workers;      // waves sharing the tile stream
    float qk_scale_log2;  // scale * k_scale * log2(e)
    float v_scale;
    int* counters;        // [S][H_kv], zero on entry and on exit
    float* slots;         // [2 * num_workers][GM * (D + 2)]
    void* out;
};

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kWavesPerGroup = 4;
constexpr int kThreads = kWavesPerGroup * kWave;
constexpr int kPrefetch = 1;  // tiles whose K and V a wave has in flight

template <int KT, int D>
struct DecodeShape {
    static constexpr int kLanesPerRow = D / kElemsPerLane;          // 16 (D=128) or 8 (D=64)
    static constexpr int kRowsPerInst = kWave / kLanesPerRow;        // 4 or 8
    static constexpr int kInstPerTile = kBlock / kRowsPerInst;       // 4 or 2
};

// Query registers: 8 elements per head, kept packed for the dot2 paths.
template <int QT, int KT>
struct QRegs;

template <>
struct QRegs<PKV_F16, PKV_F16> {
    half2_t v[4];
    __device__ __forceinline__ void load(const uint8_t* p) {
        uint4 a = *reinterpret_cast<const uint4*>(p);
        v[0] = __builtin_bit_cast(half2_t, a.x);
        v[1] = __builtin_bit_cast(half2_t, a.y);
        v[2] = __builtin_bit_cast(half2_t, a.z);
        v[3] = __builtin_bit_cast(half2_t, a.w);
    }
    __device__ __forceinline__ void zero() {
        for (int i = 0; i < 4; ++i) v[i] = half2_t{0, 0};
    }
    __device__ __forceinline__ float dot(const Chunk<PKV_F16>& k) const {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.w[i]), v[i], acc, false);
        return acc;
    }
};

template <>
struct QRegs<PKV_BF16, PKV_BF16> {
    bf162_t v[4];
    __device__ __forceinline__ void load(const uint8_t* p) {
        uint4 a = *reinterpret_cast<const uint4*>(p);
        v[0] = __builtin_bit_cast(bf162_t, a.x);
        v[1] = __builtin_bit_cast(bf162_t, a.y);
        v[2] = __builtin_bit_cast(bf162_t, a.z);
        v[3] = __builtin_bit_cast(bf162_t, a.w);
    }
    __device__ __forceinline__ void zero() {
        for (int i = 0; i < 4; ++i) v[i] = __builtin_bit_cast(bf162_t, 0u);
    }
    __device__ __forceinline__ float dot(const Chunk<PKV_BF16>& k) const {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.w[i]), v[i], acc,
                                                  false);
        return acc;
    }
};

// float32 query over float32 caches.
template <>
struct QRegs<PKV_F32, PKV_F32> {
    float v[8];
    __device__ __forceinline__ void load(const uint8_t* p) {
        Chunk<PKV_F32> c = load_chunk<PKV_F32>(p);
        chunk_to_f32<PKV_F32>(c, v);
    }
    __device__ __forceinline__ void zero() {
        for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    __device__ __forceinline__ float dot(const Chunk<PKV_F32>& k) const {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = fmaf(v[i], __builtin_bit_cast(float, k.w[i]), acc);
        return acc;
    }
};

// 16-bit query over an fp8 cache: the 8 codes of a chunk are widened to the
// query's type (exact: every E4M3 value is a bf16 and an f16 value; the
// scaled conversions run with scale 1), then the same dot2 path.
template <>
struct QRegs<PKV_BF16, PKV_FP8_E4M3> : QRegs<PKV_BF16, PKV_BF16> {
    __device__ __forceinline__ float dot(const Chunk<PKV_FP8_E4M3>& k) const {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const bf162_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k.w[i], 1.0f, false);
            const bf162_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k.w[i], 1.0f, true);
            acc = __builtin_amdgcn_fdot2_f32_bf16(lo, v[2 * i], acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(hi, v[2 * i + 1], acc, false);
        }
        return acc;
    }
};

template <>
struct QRegs<PKV_F16, PKV_FP8_E4M3> : QRegs<PKV_F16, PKV_F16> {
    __device__ __forceinline__ float dot(const Chunk<PKV_FP8_E4M3>& k) const {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k.w[i], 1.0f, false);
            const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k.w[i], 1.0f, true);
            acc = __builtin_amdgcn_fdot2(lo, v[2 * i], acc, false);
            acc = __builtin_amdgcn_fdot2(hi, v[2 * i + 1], acc, false);
        }
        return acc;
    }
};

// Scores are kept in log2 units; a wave only rescales its running sums when a
// new score exceeds its running max by more than kLazyRescale (2^8 headroom
// for the unnormalised weights, far inside float32 range). The result is the
// same softmax: every weight is exp2(x - m) against one common m per wave.
constexpr float kLazyRescale = 8.0f;

__device__ __forceinline__ int tiles_of(int n, int max_ctx) {
    return (n > 0 && n <= max_ctx) ? (n + kBlock - 1) / kBlock : 0;
}

// Sum over the wave, returned as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int sh = 1; sh < kWave; sh <<= 1) v += __shfl_xor(v, sh, kWave);
    return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int u = __shfl_up(v, d, kWave);
        if (lane >= d) v += u;
    }
    return v;
}

// 8 float32 values rounded into the output type, one 16- or 32-byte store.
template <int OT>
__device__ __forceinline__ void store8(void* base, size_t idx, const float* f) {
    if constexpr (OT == PKV_F32) {
        float4* d = reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + idx);
        d[0] = make_float4(f[0], f[1], f[2], f[3]);
        d[1] = make_float4(f[4], f[5], f[6], f[7]);
    } else {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint16_t lo, hi;
            if constexpr (OT == PKV_F16) {
                lo = __builtin_bit_cast(uint16_t, (_Float16)f[2 * i]);
                hi = __builtin_bit_cast(uint16_t, (_Float16)f[2 * i + 1]);
            } else {
                lo = f32_to_bf16_rne(f[2 * i]);
                hi = f32_to_bf16_rne(f[2 * i + 1]);
            }
            w[i] = (uint32_t)lo | ((uint32_t)hi << 16);
        }
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(base) + idx) =
            make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Partials cross between waves on different XCDs (each XCD has its own L2).
// They are written and read with agent-scope atomic (write-through, coherent)
// accesses, and the writer waits for its stores to complete before it bumps
// the segment counter; no cache writeback or invalidate of a whole L2 (what a
// device-scope fence costs on this chip) is needed.
__device__ __forceinline__ void coherent_store(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A wave-uniform read of an input table the kernel never writes (block
// tables, context lengths): through the constant address space it becomes a
// scalar load, which leaves the vector-memory wait counter to the tile data.
__device__ __forceinline__ int32_t uniform_read(const int32_t* base, size_t i) {
    return ((const __attribute__((address_space(4))) int32_t*)base)[i];
}

// Everything that computes v[] happens before this point, and no memory
// access moves across it. Placed between the last read of a ring slot and the
// loads that refill it, it keeps the old and the new contents of the slot from
// being live at once, so the refill can land in the same registers.
template <int N>
__device__ __forceinline__ void settle(float (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]) : : "memory");
}

// The worker wave whose slice [a_w, a_{w+1}) holds tile f, a_w = floor(w*T/NW).
__device__ __forceinline__ int worker_of(int64_t f, int64_t total, int nw) {
    return (int)(((f + 1) * nw - 1) / total);
}

// Merge the partials of one split segment, left by workers w0..w1 (worker w0
// in its slot k0, the others in slot 0), into the output rows orow..orow+G-1:
//   M = max_j m_j,  out = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j.
// Lane j reads partial j's maxima and sums; the accumulators of 8 partials
// are in flight at a time.
template <int QT, int D, int GM>
__device__ __forceinline__ void merge_segment(const DecodeParams& p, int w0, int w1,
                                                        int k0, int G, size_t orow, int lane) {
    constexpr int SLOT = decode_slot_floats(GM, D);
    static_assert(D % kWave == 0, "head size must be a multiple of the wave width");
    constexpr int PER_LANE = GM * D / kWave;  // accumulator elements per lane
    const int nparts = w1 - w0 + 1;
    auto slot_of = [&](int j) {
        return p.slots + (size_t)(2 * (w0 + j) + (j == 0 ? k0 : 0)) * SLOT;
    };
    float mx[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) mx[h] = -INFINITY;
    for (int j0 = 0; j0 < nparts; j0 += kWave) {
        const int j = j0 + lane;
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            const float v = j < nparts ? coherent_load(slot_of(j) + GM * D + h) : -INFINITY;
            mx[h] = fmaxf(mx[h], wave_max(v));
        }
    }
    float lsum[GM], o[PER_LANE];
#pragma unroll
    for (int h = 0; h < GM; ++h) lsum[h] = 0.f;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) o[i] = 0.f;
    for (int j0 = 0; j0 < nparts; j0 += kWave) {
        const int j = j0 + lane;
        float c[GM];
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            const float* sl = slot_of(min(j, nparts - 1));
            c[h] = j < nparts ? __builtin_amdgcn_exp2f(coherent_load(sl + GM * D + h) - mx[h]) : 0.f;
            lsum[h] += wave_sum(j < nparts ? coherent_load(sl + GM * D + GM + h) * c[h] : 0.f);
        }
        const int cnt = min(kWave, nparts - j0);
#pragma unroll 8
        for (int jj = 0; jj < cnt; ++jj) {
            const float* sl = slot_of(j0 + jj);
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i) {
                const int idx = i * kWave + lane;       // h * D + e
                if (idx < GM * D) {
                    // D is a multiple of the wave width, so the head of
                    // element idx is (i * kWave) / D: known at compile time
                    const int cj = __builtin_amdgcn_readlane(
                        __builtin_bit_cast(int, c[(i * kWave) / D]), jj);
                    o[i] = fmaf(__builtin_bit_cast(float, cj), coherent_load(sl + idx), o[i]);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const int idx = i * kWave + lane;
        const int h = (i * kWave) / D, e = idx % D;
        if (idx < GM * D && h < G) store_f32_as<QT>(p.out, (orow + h) * D + e, o[i] * (p.v_scale / lsum[h]));
    }
}

template <int KT, int QT, int D, int GM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void paged_decode_kernel(DecodeParams p) {
    using Shape = DecodeShape<KT, D>;
    constexpr int LPR = Shape::kLanesPerRow;
    constexpr int RPI = Shape::kRowsPerInst;
    constexpr int NI = Shape::kInstPerTile;
    constexpr int KB = Elem<KT>::bytes;
    constexpr int QB = Elem<QT>::bytes;
    constexpr int ROW_BYTES = D * KB;
    constexpr int SLOT = decode_slot_floats(GM, D);

    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kWavesPerGroup) + wave_id());
    const int nw_launch = p.num_workers;
    if (w >= nw_launch) return;
    const int S = p.num_seqs, H = p.num_kv_heads, G = p.group, Hq = p.num_q_heads;
    const int mb = p.max_blocks_per_seq;
    const int max_ctx = mb * kBlock;
    const float nan = __builtin_nanf("");

    // Sequences with no tiles: a zero row (n <= 0) or a NaN row (n longer than
    // the block-table row). One wave writes each.
    for (int s = w; s < S; s += nw_launch) {
        const int n = p.context_lens[s];
        if (n > 0 && n <= max_ctx) continue;
        const float fill = n <= 0 ? 0.f : nan;
        for (int idx = lane; idx < Hq * D; idx += kWave)
            store_f32_as<QT>(p.out, (size_t)s * Hq * D + idx, fill);
    }

    // Total tiles T and this wave's slice.
    int64_t total = 0;
    for (int base = 0; base < S; base += kWave) {
        const int s = base + lane;
        total += wave_sum_int(s < S ? tiles_of(p.context_lens[s], max_ctx) : 0);
    }
    total *= H;
    if (total == 0) return;
    const int nw = (int)min((int64_t)nw_launch, total);  // every slice non-empty
    if (w >= nw) return;
    const int64_t a = (int64_t)w * total / nw;
    const int64_t b = (int64_t)(w + 1) * total / nw;

    // The sequence holding tile a, and the number of tiles before it.
    int cs = 0;
    int64_t seq_base = 0;
    {
        int64_t before = 0;
        for (int base = 0; base < S; base += kWave) {
            const int s = base + lane;
            const int t = s < S ? tiles_of(p.context_lens[s], max_ctx) * H : 0;
            const int incl = wave_inclusive_scan(t, lane);
            const int64_t lo = before + incl - t;
            const unsigned long long hit = __ballot(t > 0 && lo <= a && a < before + incl);
            if (hit) {
                const int L = __ffsll(hit) - 1;
                cs = base + L;
                seq_base = before + __builtin_amdgcn_readlane(incl - t, L);
                break;
            }
            before += __builtin_amdgcn_readlane(incl, kWave - 1);
        }
    }

    // A position in the tile stream: segment (s, g) of sequence length n and
    // nb tiles whose first tile has index seg; block bi; the wave's slice of
    // the segment ends at block hi. All fields are wave-uniform.
    struct Cursor {
        int s, g, n, nb, bi, hi;
        int64_t seg;
    };
    // Move c to the first block of the next segment (order s, then g) inside
    // the slice; false when the slice has no more tiles.
    auto next_segment = [&](Cursor& c) -> bool {
        const int64_t seg = c.seg + c.nb;
        if (seg >= b) return false;
        if (c.g + 1 < H) {
            ++c.g;
        } else {
            int s = c.s + 1, n = 0, nb = 0;
            for (; s < S; ++s) {
                n = uniform_read(p.context_lens, s);
                nb = tiles_of(n, max_ctx);
                if (nb > 0) break;
            }
            if (s >= S) return false;  // cannot happen: tiles after seg exist
            c.s = s;
            c.g = 0;
            c.n = n;
            c.nb = nb;
        }
        c.seg = seg;
        c.bi = 0;
        c.hi = (int)min((int64_t)c.nb, b - seg);
        return true;
    };

    Cursor cc;  // the tile being computed
    cc.s = cs;
    cc.n = uniform_read(p.context_lens, cs);
    cc.nb = tiles_of(cc.n, max_ctx);
    if (cc.nb == 0) return;  // cannot happen: tile a lies in a non-empty sequence
    cc.g = (int)((a - seq_base) / cc.nb);
    cc.bi = (int)((a - seq_base) % cc.nb);
    cc.seg = seq_base + (int64_t)cc.g * cc.nb;
    cc.hi = (int)min((int64_t)cc.nb, cc.bi + (b - a));
    int clo = cc.bi;           // first block of the computed piece
    bool first_piece = true;   // the piece holding tile a (partial slot 0)
    bool piece_bad = false;

    Cursor ic = cc;  // the next tile to load (kPrefetch tiles ahead of cc)
    bool ic_valid = true;
    // Block id of ic's tile, read with a wave-uniform (scalar) load one tile
    // before it is needed; -1 marks an id outside the pool. Scalar loads keep
    // the tile loads' wait counter free of anything but tile data.
    auto read_id = [&](const Cursor& c) -> int {
        const int id = uniform_read(p.block_tables, (size_t)c.s * mb + c.bi);
        return (id < 0 || id >= p.num_blocks) ? -1 : id;
    };
    int ic_id = read_id(ic);
    auto ic_advance = [&]() {
        if (!ic_valid) return;
        if (++ic.bi == ic.hi) ic_valid = next_segment(ic);
        if (ic_valid) ic_id = read_id(ic);
    };

    const int row = lane / LPR;                        // which of the RPI rows
    const int col = (lane % LPR) * kElemsPerLane;      // first element this lane owns

    QRegs<QT, KT> qr[GM];
    auto load_q = [&](int s, int g) {
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            if (h < G)
                qr[h].load(p.q + (((size_t)s * Hq + g * G + h) * D + col) * QB);
            else
                qr[h].zero();
        }
    };

    // tile base (wave-uniform, scalar registers) + this lane's byte offset
    const uint32_t lane_off = (uint32_t)(row * ROW_BYTES + col * KB);
    Chunk<KT> kr[kPrefetch][NI], vr[kPrefetch][NI];
    bool slot_bad[kPrefetch];
    // Where ic's tile lives, and how many of its bytes to read: a whole tile,
    // or none once the slice is exhausted or the block id is outside the pool
    // (such a tile's piece is written as NaN). Every iteration issues the
    // same loads either way, which keeps the compiler's memory waits exact;
    // a load past a buffer resource's size returns zeros without touching
    // memory.
    struct TileRef {
        size_t off;
        uint32_t bytes;
    };
    auto ic_tile = [&](bool& bad_tile) -> TileRef {
        bad_tile = ic_valid && ic_id < 0;
        if (!ic_valid || ic_id < 0) return TileRef{0, 0u};
        return TileRef{cache_row_offset(ic_id, ic.g, 0, H, ROW_BYTES),
                       (uint32_t)(kBlock * ROW_BYTES)};
    };
    // Each tile is read through its own buffer resource (base = the tile,
    // 16 rows), nontemporal: every cache byte is used once per call. The
    // scheduling barriers keep a refill after the last read of the slot it
    // overwrites, so the ring registers stay put from one pass to the next
    // (no copies of data still in flight).
    auto issue_k = [&](int slot, TileRef t_) {
        const __amdgpu_buffer_rsrc_t t = make_rsrc(p.k_cache + t_.off, t_.bytes);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < NI; ++r)
            kr[slot][r] = load_chunk_stream<KT>(t, lane_off + r * RPI * ROW_BYTES);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto issue_v = [&](int slot, TileRef t_) {
        const __amdgpu_buffer_rsrc_t t = make_rsrc(p.v_cache + t_.off, t_.bytes);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < NI; ++r)
            vr[slot][r] = load_chunk_stream<KT>(t, lane_off + r * RPI * ROW_BYTES);
        __builtin_amdgcn_sched_barrier(0);
    };

    // The query first: the oldest load in flight, so the first tile's wait
    // covers it and the loop never has to wait for everything.
    load_q(cc.s, cc.g);
#pragma unroll
    for (int slot = 0; slot < kPrefetch; ++slot) {
        const TileRef t = ic_tile(slot_bad[slot]);
        issue_k(slot, t);
        issue_v(slot, t);
        ic_advance();
    }

    float m[GM], l[GM], acc[GM][kElemsPerLane];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < kElemsPerLane; ++e) acc[h][e] = 0.f;
    }
    const float qk_scale = p.qk_scale_log2;
    bool active = true;  // cc holds a tile still to compute

    // Split segments whose partials this wave was the last to deliver. Only
    // the first and the last piece of a slice can be partial, so there are at
    // most two; they are merged after the stream, which keeps the merge's
    // loads and registers out of the streaming loop.
    struct Pending {
        int s, g, nb;
        int64_t seg;
    };
    Pending pend0{}, pend1{};
    int npend = 0;

    // Every pass of the loop computes one tile per ring slot and issues the
    // loads that refill the slot, unconditionally: a pass after the last
    // tile only re-reads and computes on data nobody keeps. Only the piece
    // bookkeeping depends on `active`. One back edge with the same loads on
    // every path lets the compiler wait for exactly the tile it needs.
    while (active) {
#pragma unroll
        for (int slot = 0; slot < kPrefetch; ++slot) {
            piece_bad |= slot_bad[slot];
            bool next_bad;
            const TileRef nxt = ic_tile(next_bad);

            // ---- one row instruction at a time: QK, online softmax, P.V ----
            // The next K goes out once the last QK has read this slot's K, the
            // next V once the last P.V has read this slot's V.
            const int live_rows = cc.n - cc.bi * kBlock;   // rows < live_rows hold positions < n
#pragma unroll
            for (int r = 0; r < NI; ++r) {
                const bool live = r * RPI + row < live_rows;
                float x[GM];
#pragma unroll
                for (int h = 0; h < GM; ++h) {
                    x[h] = group_sum<LPR>(qr[h].dot(kr[slot][r])) * qk_scale;
                    x[h] = live ? x[h] : -INFINITY;
                }
                if (r == NI - 1) {
                    settle(x);
                    issue_k(slot, nxt);
                }
#pragma unroll
                for (int h = 0; h < GM; ++h) {
                    if (__any(x[h] > m[h] + kLazyRescale)) {
                        float bm = x[h];
#pragma unroll
                        for (int sh = LPR; sh < kWave; sh <<= 1) bm = fmaxf(bm, __shfl_xor(bm, sh, kWave));
                        const float mn = fmaxf(m[h], bm);
                        const float c = __builtin_amdgcn_exp2f(m[h] - mn);
                        l[h] *= c;
#pragma unroll
                        for (int e = 0; e < kElemsPerLane; ++e) acc[h][e] *= c;
                        m[h] = mn;
                    }
                }
                float vf[kElemsPerLane];
                chunk_to_f32<KT>(vr[slot][r], vf);
#pragma unroll
                for (int e = 0; e < kElemsPerLane; ++e) vf[e] = live ? vf[e] : 0.f;
                if (r == NI - 1) settle(vf);
#pragma unroll
                for (int h = 0; h < GM; ++h) {
                    const float pr = __builtin_amdgcn_exp2f(x[h] - m[h]);
                    l[h] += pr;
#pragma unroll
                    for (int e = 0; e < kElemsPerLane; ++e) acc[h][e] = fmaf(pr, vf[e], acc[h][e]);
                }
            }
            issue_v(slot, nxt);
            slot_bad[slot] = next_bad;
            ic_advance();

            if (!active) continue;
            if (cc.bi + 1 < cc.hi) {
                ++cc.bi;
                continue;
            }

            // ---- the piece is done: write it out, or leave a partial ----
            // Sum the rows of the wave (lanes with equal `col` hold different rows).
#pragma unroll
            for (int h = 0; h < GM; ++h) {
#pragma unroll
                for (int sh = LPR; sh < kWave; sh <<= 1) l[h] += __shfl_xor(l[h], sh, kWave);
#pragma unroll
                for (int e = 0; e < kElemsPerLane; ++e) {
                    float v = acc[h][e];
#pragma unroll
                    for (int sh = LPR; sh < kWave; sh <<= 1) v += __shfl_xor(v, sh, kWave);
                    acc[h][e] = v;
                }
            }
            const size_t orow = (size_t)cc.s * Hq + (size_t)cc.g * G;  // first output row
            if (clo == 0 && cc.hi == cc.nb) {
                // the whole segment: normalise and store
                if (lane < LPR) {
#pragma unroll
                    for (int h = 0; h < GM; ++h) {
                        if (h >= G) break;
                        float o[kElemsPerLane];
                        const float sc = p.v_scale / l[h];
#pragma unroll
                        for (int e = 0; e < kElemsPerLane; ++e) o[e] = piece_bad ? nan : acc[h][e] * sc;
                        store8<QT>(p.out, (orow + h) * D + col, o);
                    }
                }
            } else {
                // partial of a split segment: unnormalised accumulator, max, sum
                float* slotp = p.slots + (size_t)(2 * w + (first_piece ? 0 : 1)) * SLOT;
                if (lane < LPR) {
#pragma unroll
                    for (int h = 0; h < GM; ++h)
#pragma unroll
                        for (int e = 0; e < kElemsPerLane; ++e)
                            coherent_store(slotp + h * D + col + e, acc[h][e]);
                }
                if (lane == 0) {
#pragma unroll
                    for (int h = 0; h < GM; ++h) {
                        coherent_store(slotp + GM * D + h, piece_bad ? nan : m[h]);
                        coherent_store(slotp + GM * D + GM + h, piece_bad ? nan : l[h]);
                    }
                }
                __builtin_amdgcn_s_waitcnt(0);  // the partial has landed before it is announced
                int* counter = p.counters + (size_t)cc.s * H + cc.g;
                int old = 0;
                if (lane == 0)
                    old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                old = __builtin_amdgcn_readfirstlane(old);
                const int w0 = worker_of(cc.seg, total, nw);
                const int w1 = worker_of(cc.seg + cc.nb - 1, total, nw);
                if (old == w1 - w0) {  // every partial of the segment is in
                    const Pending pd{cc.s, cc.g, cc.nb, cc.seg};
                    if (npend == 0) pend0 = pd; else pend1 = pd;
                    ++npend;
                }
            }

            // ---- next piece (its first tiles are already in flight) ----
            if (!next_segment(cc)) {
                active = false;
                continue;
            }
            clo = 0;
            first_piece = false;
            piece_bad = false;
            load_q(cc.s, cc.g);
            // The query has landed before this path joins the streaming one,
            // so the join does not make every tile wait for all loads.
            __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
            for (int h = 0; h < GM; ++h) {
                m[h] = -INFINITY;
                l[h] = 0.f;
#pragma unroll
                for (int e = 0; e < kElemsPerLane; ++e) acc[h][e] = 0.f;
            }
        }
    }

    // Merge the split segments this wave completed (log-sum-exp over the
    // partials) and leave their counters at zero for the next call.
    for (int i = 0; i < npend; ++i) {
        const Pending& pd = i == 0 ? pend0 : pend1;
        const int w0 = worker_of(pd.seg, total, nw);
        const int w1 = worker_of(pd.seg + pd.nb - 1, total, nw);
        const int k0 = (int64_t)w0 * total / nw < pd.seg ? 1 : 0;
        merge_segment<QT, D, GM>(p, w0, w1, k0, G, (size_t)pd.s * Hq + (size_t)pd.g * G, lane);
        if (lane == 0)
            __hip_atomic_store(p.counters + (size_t)pd.s * H + pd.g, 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---- dispatch ------------------------------------------------------------------

template <int KT, int QT, int D, int GM>
static hipError_t launch_typed(const DecodeArgs& a) {
    auto kernel = paged_decode_kernel<KT, QT, D, GM>;
    int nw = a.num_workers;
    if (nw == 0) {
        // fill the device: resident workgroups per CU x CUs x 4 waves
        static std::atomic<int> per_cu_cache{0};
        int per_cu = per_cu_cache.load(std::memory_order_relaxed);
        if (per_cu == 0) {
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) !=
                    hipSuccess ||
                per_cu <= 0)
                per_cu = 1;
            per_cu_cache.store(per_cu, std::memory_order_relaxed);
        }
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return hipErrorInvalidDevice;
        // two workgroups (8 waves) per CU: measured best on the 40 x 8192 GQA
        // shape; more waves only add contention for the vector ALUs
        nw = (per_cu < 2 ? per_cu : 2) * cus * kWavesPerGroup;
        if (nw > kMaxWorkers) nw = kMaxWorkers;
    }
    // never more workers than tiles could exist
    const int64_t tile_bound = (int64_t)a.num_seqs * a.num_kv_heads * a.max_blocks_per_seq;
    if (nw > tile_bound) nw = (int)tile_bound;
    if (nw < 1) nw = 1;

    DecodeParams p;
    p.q = static_cast<const uint8_t*>(a.q);
    p.k_cache = static_cast<const uint8_t*>(a.k_cache);
    p.v_cache = static_cast<const uint8_t*>(a.v_cache);
    p.block_tables = a.block_tables;
    p.context_lens = a.context_lens;
    p.num_seqs = a.num_seqs;
    p.num_q_heads = a.num_q_heads;
    p.num_kv_heads = a.num_kv_heads;
    p.group = a.group;
    p.num_blocks = a.num_blocks;
    p.max_blocks_per_seq = a.max_blocks_per_seq;
    p.num_workers = nw;
    p.qk_scale_log2 = a.scale * (KT == PKV_FP8_E4M3 ? a.k_scale : 1.f) * kLog2e;
    p.v_scale = KT == PKV_FP8_E4M3 ? a.v_scale : 1.f;
    p.counters = a.counters;
    p.slots = a.slots;
    p.out = a.out;
    const int grid = (nw + kWavesPerGroup - 1) / kWavesPerGroup;
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, a.stream, p);
    return hipGetLastError();
}

template <int KT, int QT, int D>
static hipError_t launch_group(const DecodeArgs& a) {
    switch (padded_group(a.group)) {
    case 1: return launch_typed<KT, QT, D, 1>(a);
    case 2: return launch_typed<KT, QT, D, 2>(a);
    case 4: return launch_typed<KT, QT, D, 4>(a);
    case 6: return launch_typed<KT, QT, D, 6>(a);
    default: return launch_typed<KT, QT, D, 8>(a);
    }
}

template <int KT, int QT>
static hipError_t launch_dim(const DecodeArgs& a) {
    return a.head_dim == 64 ? launch_group<KT, QT, 64>(a) : launch_group<KT, QT, 128>(a);
}

hipError_t launch_paged_decode(const DecodeArgs& a) {
    if (a.kv_dtype == PKV_F32) return launch_dim<PKV_F32, PKV_F32>(a);
    if (a.kv_dtype == PKV_F16) return launch_dim<PKV_F16, PKV_F16>(a);
    if (a.kv_dtype == PKV_BF16) return launch_dim<PKV_BF16, PKV_BF16>(a);
    if (a.q_dtype == PKV_F16) return launch_dim<PKV_FP8_E4M3, PKV_F16>(a);
    return launch_dim<PKV_FP8_E4M3, PKV_BF16>(a);
}

}  // namespace pkv
