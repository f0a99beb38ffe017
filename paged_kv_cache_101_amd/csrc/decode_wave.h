// decode_wave.h -- the decode attention of one worker wave, for gfx950 (CDNA4).
//
// What is computed (ttlab page, sections 2 and 4; drpranayjha page, "How
// PagedAttention pages the KV cache"; tarundecipher page, "Batching does not
// merge the conversations"): one query token per sequence attends over the
// sequence's own K/V rows, found through its block table in a shared pool of
// 16-token physical blocks; a group of G query heads shares one KV head.
//
// Work decomposition: a persistent, evenly split tile stream
//   * A "tile" is one (sequence s, KV head g, logical block b): 16 tokens of K
//     and of V, D elements each, contiguous in the pool. All tiles of the
//     batch are numbered s-major, then g, then b. Each worker wave takes an
//     equal contiguous slice of that numbering (within one tile of every other
//     wave), whatever the mix of sequence lengths.
//   * A wave streams its slice: the next tile's K is in flight while the
//     current tile's scores and softmax are computed, its V while the current
//     P.V runs. Cache tiles use nontemporal loads (read once).
//   * A slice covers whole (s, g) segments and at most two partial ones. A
//     segment finished by one wave is written out directly. A segment split
//     over several waves (the split-KV case) leaves one partial (running max
//     m, sum l, unnormalised accumulator) per wave in the workspace; the last
//     wave to finish the segment, found with a device-scope counter, merges
//     them with the log-sum-exp rule and writes the output.
//   * Fixed partitions (PART, the caller's partition_size): the unit of the
//     split is a partition of partition_size / 16 tiles instead of a tile,
//     each wave takes whole partitions, every piece ends at a partition end,
//     and each partition of a multi-partition segment leaves its partial in
//     its own workspace slot; partition_merge_kernel, launched next on the
//     stream, reduces them by the log-sum-exp rule.
//
// Per tile, both contractions run on the matrix cores, in the operand layouts
// of the 16x16 MFMA shapes (lane l: column/row l % 16, k-group l / 16):
//   * QK^T as S^T = K_tile (16 tokens x D) . Q^T (D x 16 head columns, the G
//     query heads of the KV head, zero-padded): D/32 MFMA 16x16x32 (16-bit),
//     each lane feeding one token's 8-element K slab straight from its load.
//     Lane l ends with the scores of head l % 16 for tokens 4*(l/16) + j.
//   * Those four scores per lane are exactly the A operand of P.V:
//     O (16 heads x D) += P (16 x 16 tokens) . V_tile (16 tokens x D), as D/16
//     MFMA 16x16x16 whose B operand is 4 tokens of one element row of V,
//     again straight from the load (V is stored element-major in the tile).
//   * Softmax is online in log2 units with a lazily moved maximum: the scores
//     of a tile only trigger a rescale (a wave-uniform branch with the
//     cross-lane max) when one exceeds the running max by more than 8.
//   * P is rounded to the query's 16-bit type for the P.V operand, and the sum
//     l accumulates the rounded weights, so the output is an exactly
//     normalised average. float32 caches use the float32 MFMA (16x16x4) and
//     keep P in float32. fp8 K/V are widened exactly to the query's type.
// Positions >= n inside a sequence's last block are excluded by select
// (score -inf, V element zero), never by arithmetic, so garbage or NaN there
// cannot leak.
//
// Suffix pass of the shared-prefix decode (PFX): a sequence in a prefix group
// streams only the blocks after its group's shared ones, and its rows go to a
// float32 result (the normalised output without v_scale, and the
// log2-sum-exp of its scores) that the prefix pass merges with the prefix's
// partials (paged_prefill.hip, prefix mode). Other sequences are decoded as usual.
#pragma once

#include "pkv_internal.h"
#include "pkv_tile.h"

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
    // fixed partitions (PART): partition_size / 16 tiles per partition, and
    // partition slots per (sequence, KV head) segment in the workspace
    int part_tiles;
    int part_stride;
    float qk_scale_log2;  // scale * k_scale * log2(e)
    float v_scale;
    int* counters;        // [S][H_kv], zero on entry and on exit
    float* slots;         // balanced: [2 * num_workers][SLOT]; PART: [S][H_kv][part_stride][SLOT]
    void* out;
    // suffix pass only (PFX): the prefix-group description and the float32
    // results of grouped sequences
    int num_groups;
    const int32_t* group_starts;  // [num_groups + 1]
    const int32_t* group_prefix;  // [num_groups]
    float* res_o;                 // [S][H_q][D]: acc / l
    float* res_lse;               // [S][H_q]: m + log2(l), log2 units of the scores
};

constexpr int kWavesPerGroup = 1;  // one worker wave per workgroup: any count spreads evenly
constexpr int kThreads = kWavesPerGroup * kWave;
constexpr int kPrefetch = 1;  // tiles whose K and V a wave has in flight

// Tiles of a sequence of n tokens whose first `pre` blocks are left out
// (pre = 0: all of them). A length outside (0, max_ctx] has none.
__device__ __forceinline__ int tiles_of(int n, int pre, int max_ctx) {
    if (n <= 0 || n > max_ctx) return 0;
    const int m = n - pre * kBlock;
    return m > 0 ? (m + kBlock - 1) / kBlock : 0;
}

// Write a float32 suffix result for rows (s, h), h < Hq, with no suffix
// tiles: empty (n == 16 * pre: weight zero) or not valid (NaN).
template <int D>
__device__ __forceinline__ void write_empty_result(const DecodeParams& p, int s, bool empty,
                                                   int lane) {
    const int Hq = p.num_q_heads;
    const float o = empty ? 0.f : __builtin_nanf("");
    for (int idx = lane; idx < Hq * D; idx += kWave) p.res_o[(size_t)s * Hq * D + idx] = o;
    for (int h = lane; h < Hq; h += kWave) p.res_lse[(size_t)s * Hq + h] = empty ? -INFINITY : o;
}

// The worker wave whose slice [a_w, a_{w+1}) holds tile f, a_w = floor(w*T/NW).
__device__ __forceinline__ int worker_of(int64_t f, int64_t total, int nw) {
    return (int)(((f + 1) * nw - 1) / total);
}

// Merge the nparts partials of one split segment (partial j at slot_of(j))
// into the output rows orow..orow+G-1:
//   M = max_j m_j,  out = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j.
// With at most 64 partials (the usual case), lane j reads partial j's maxima
// and sums, and in the same memory round every lane reads its accumulator
// elements of the first KPRE partials, so a merge of up to KPRE partials
// waits for one round trip (it runs on the launch's tail, where each round
// trip to memory shows); later partials follow, several in flight at a time.
// With more than 64 partials, the maxima and sums are read in passes of 64
// partials and one partial's accumulators are in flight at a time.
template <int QT, int D, int GM, typename SlotOf>
__device__ __forceinline__ void merge_segment(const DecodeParams& p, int nparts, SlotOf slot_of,
                                              int G, size_t orow, int lane, bool to_result) {
    static_assert(D % kWave == 0, "head size must be a multiple of the wave width");
    constexpr int PER_LANE = GM * D / kWave;  // accumulator elements per lane
    // partials read with the maxima: up to 16, about 128 registers of
    // accumulators (a default launch keeps at most two waves per SIMD, so
    // registers are not what limits it)
    constexpr int KPRE = 128 / PER_LANE > 16 ? 16 : 128 / PER_LANE;
    float mx[GM];
    float lsum[GM], o[PER_LANE];
#pragma unroll
    for (int h = 0; h < GM; ++h) lsum[h] = 0.f;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) o[i] = 0.f;
    if (nparts <= kWave) {
        // At most one partial per lane: its maxima and sums are read once,
        // together with the accumulators of the first KPRE partials.
        const int j = min(lane, nparts - 1);
        const float* sl = slot_of(j);
        float mj[GM], lj[GM];
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            mj[h] = lane < nparts ? coherent_load(sl + GM * D + h) : -INFINITY;
            lj[h] = lane < nparts ? coherent_load(sl + GM * D + GM + h) : 0.f;
        }
        float pre[KPRE][PER_LANE];
#pragma unroll
        for (int k = 0; k < KPRE; ++k) {
            if (k < nparts) {  // wave-uniform
                const float* sk = slot_of(k);
#pragma unroll
                for (int i = 0; i < PER_LANE; ++i) {
                    const int idx = i * kWave + lane;  // h * D + e
                    pre[k][i] = idx < GM * D ? coherent_load(sk + idx) : 0.f;
                }
            }
        }
        float c[GM];
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            mx[h] = wave_max(mj[h]);
            c[h] = lane < nparts ? __builtin_amdgcn_exp2f(mj[h] - mx[h]) : 0.f;
            lsum[h] = wave_sum(lj[h] * c[h]);
        }
        // partial k's weights sit in lane k
#pragma unroll
        for (int k = 0; k < KPRE; ++k) {
            if (k < nparts) {
#pragma unroll
                for (int i = 0; i < PER_LANE; ++i) {
                    const float wk = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c[(i * kWave) / D]), k));
                    o[i] = fmaf(wk, pre[k][i], o[i]);
                }
            }
        }
        // Later partials: every lane forms partial jj's weights itself from
        // its maxima (one address for the whole wave), so the loop holds no
        // cross-lane read and unrolls: the loads of four partials (two with
        // 16 accumulator elements per lane, where four measured 30% slower)
        // are in flight at a time.
        constexpr int kMergeUnroll = PER_LANE <= 12 ? 4 : 2;
#pragma unroll kMergeUnroll
        for (int jj = KPRE; jj < nparts; ++jj) {
            const float* sj = slot_of(jj);
            float wj[GM];
#pragma unroll
            for (int h = 0; h < GM; ++h) wj[h] = __builtin_amdgcn_exp2f(coherent_load(sj + GM * D + h) - mx[h]);
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i) {
                const int idx = i * kWave + lane;  // h * D + e
                if (idx < GM * D) o[i] = fmaf(wj[(i * kWave) / D], coherent_load(sj + idx), o[i]);
            }
        }
    } else {
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
    }
    if (to_result) {
        // suffix pass: the normalised rows and their log2-sum-exp, float32
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
            const int idx = i * kWave + lane;
            const int h = (i * kWave) / D, e = idx % D;
            if (idx < GM * D && h < G) p.res_o[(orow + h) * D + e] = o[i] / lsum[h];
        }
#pragma unroll
        for (int h = 0; h < GM; ++h)
            if (h < G && lane == 0) p.res_lse[orow + h] = mx[h] + __log2f(lsum[h]);
        return;
    }
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
        const int idx = i * kWave + lane;
        const int h = (i * kWave) / D, e = idx % D;
        if (idx < GM * D && h < G) store_f32_as<QT>(p.out, (orow + h) * D + e, o[i] * (p.v_scale / lsum[h]));
    }
}

// One worker wave of the decode launch: wave w of p.num_workers (waves at or
// past it return at once). The decode kernel runs one per workgroup; the
// shared-prefix call's fused launch runs four per workgroup beside its
// prefix-pass workgroups.
template <int KT, int QT, int D, int GM, bool PFX, bool PART>
__device__ __forceinline__ void decode_wave(const DecodeParams& p, int w) {
    using TM = TileMath<KT, QT, D>;
    constexpr int NK = TM::NK, NV = TM::NV, NVL = TM::NVL, KW = TM::KW, VLW = TM::VLW;
    constexpr int KB = Elem<KT>::bytes;
    constexpr int QB = Elem<QT>::bytes;
    constexpr uint32_t kTileBytes = (uint32_t)kBlock * D * KB;
    constexpr int SLOT = decode_slot_floats(GM, D);
    static_assert(!(PFX && PART), "the suffix pass uses the balanced split");

    const int lane = lane_id();
    const int nw_launch = p.num_workers;
    if (w >= nw_launch) return;
    const int S = p.num_seqs, H = p.num_kv_heads, G = p.group, Hq = p.num_q_heads;
    const int mb = p.max_blocks_per_seq;
    const int max_ctx = mb * kBlock;
    const int pt = PART ? p.part_tiles : 1;  // tiles per partition (PART)
    const float nan = __builtin_nanf("");
    // The lengths of the first kScanChunks * 64 sequences, read once (one
    // memory round, with the prefix groups' description) and kept in
    // registers: the scan, the sequences with no tiles and every segment
    // change of the tile stream take them from here.
    constexpr int kScanChunks = 4;
    constexpr int kCached = kScanChunks * kWave;
    int n_c[kScanChunks], u_c[kScanChunks];  // length and units of sequence c * 64 + lane
#pragma unroll
    for (int c = 0; c < kScanChunks; ++c) {
        const int s = c * kWave + lane;
        n_c[c] = s < S ? p.context_lens[s] : 0;
    }
    // Prefix groups (suffix pass only; an unusable description counts as
    // none). Up to 64 groups are held one per lane, start, end and shared
    // blocks of group `lane`, so that finding a sequence's group takes no
    // memory round; more are searched in memory.
    int ng = 0, g_a = 0, g_b = 0, g_p = 0;
    if constexpr (PFX) {
        const int ngd = p.num_groups;
        if (ngd > 0 && ngd <= kWave) {
            bool ok = true;
            if (lane < ngd) {
                g_a = p.group_starts[lane];
                g_b = p.group_starts[lane + 1];
                g_p = p.group_prefix[lane];
                ok = g_a >= 0 && g_a <= g_b && g_b <= S && g_p >= 0 && g_p <= mb;
            }
            ng = __ballot(!ok) == 0 ? ngd : 0;
            if (ng == 0) g_a = g_b = 0;  // no group matches any sequence
        } else {
            ng = usable_groups(p.group_starts, p.group_prefix, ngd, S, mb, lane);
        }
    }
    const bool grp_lanes = PFX && ng > 0 && ng <= kWave;
    // shared blocks of sequence s: wave-uniform s, and s per lane
    auto pre_uniform = [&](int s) -> int {
        if constexpr (PFX) {
            if (grp_lanes) {
                const unsigned long long hit = __ballot(g_a <= s && s < g_b);
                return hit ? __builtin_amdgcn_readlane(g_p, __ffsll(hit) - 1) : 0;
            }
            return prefix_blocks_of<true>(p.group_starts, p.group_prefix, ng, s);
        } else {
            return 0;
        }
    };
    auto pre_lane = [&](int s) -> int {
        if constexpr (PFX) {
            if (grp_lanes) {
                int pre = 0;
                for (int j = 0; j < ng; ++j) {
                    const int a = __builtin_amdgcn_readlane(g_a, j), b = __builtin_amdgcn_readlane(g_b, j);
                    pre = (a <= s && s < b) ? __builtin_amdgcn_readlane(g_p, j) : pre;
                }
                return pre;
            }
            return prefix_blocks_of<false>(p.group_starts, p.group_prefix, ng, s);
        } else {
            return 0;
        }
    };
    // length of sequence s (wave-uniform)
    auto len_uniform = [&](int s) -> int {
        if (s < kCached) {
            int n = 0;
#pragma unroll
            for (int c = 0; c < kScanChunks; ++c)
                if ((s >> 6) == c) n = __builtin_amdgcn_readlane(n_c[c], s & (kWave - 1));
            return n;
        }
        return uniform_read(p.context_lens, s);
    };
    // Units of work a segment of nb tiles holds: its tiles (balanced split),
    // or its partitions of pt tiles (PART).
    auto units_of = [&](int nb) -> int {
        if constexpr (PART) return (nb + pt - 1) / pt;
        else return nb;
    };

    // Sequences with no tiles: a zero row (n <= 0) or a NaN row (n longer than
    // the block-table row). In the suffix pass a grouped sequence with no
    // suffix tiles gets an empty result (n == 16 * pre) or a NaN one (its
    // length does not hold its group's prefix). One wave writes each.
    for (int s = w; s < S; s += nw_launch) {
        const int n = len_uniform(s);
        const int pre = pre_uniform(s);
        if (tiles_of(n, pre, max_ctx) > 0) continue;
        if (PFX && pre > 0) {
            write_empty_result<D>(p, s, n == pre * kBlock, lane);
            continue;
        }
        const float fill = n <= 0 ? 0.f : nan;
        for (int idx = lane; idx < Hq * D; idx += kWave)
            store_f32_as<QT>(p.out, (size_t)s * Hq * D + idx, fill);
    }

    // Total units T and this wave's slice [a, b) of them. Units are numbered
    // like the tiles: sequence-major, then KV head, then position.
    int64_t total = 0;
#pragma unroll
    for (int c = 0; c < kScanChunks; ++c) {
        const int s = c * kWave + lane;
        u_c[c] = s < S ? units_of(tiles_of(n_c[c], pre_lane(s), max_ctx)) * H : 0;
        if (c * kWave < S) total += wave_sum_int(u_c[c]);
    }
    for (int base = kScanChunks * kWave; base < S; base += kWave) {
        const int s = base + lane;
        total += wave_sum_int(s < S ? units_of(tiles_of(p.context_lens[s], pre_lane(s), max_ctx)) * H : 0);
    }
    if (total == 0) return;
    const int nw = (int)min((int64_t)nw_launch, total);  // every slice non-empty
    if (w >= nw) return;
    const int64_t a = (int64_t)w * total / nw;
    const int64_t b = (int64_t)(w + 1) * total / nw;

    // The sequence holding unit a, its length, and the number of units before it.
    int cs = 0, cs_n = 0;
    int64_t seq_base = 0;
    {
        int64_t before = 0;
        for (int base = 0; base < S; base += kWave) {
            const int s = base + lane;
            const int ci = base / kWave;
            int n = 0, t = 0;
            if (ci < kScanChunks) {
#pragma unroll
                for (int c = 0; c < kScanChunks; ++c)
                    if (c == ci) n = n_c[c], t = u_c[c];
            } else if (s < S) {
                n = p.context_lens[s];
                t = units_of(tiles_of(n, pre_lane(s), max_ctx)) * H;
            }
            const int incl = wave_inclusive_scan(t);
            const int64_t lo = before + incl - t;
            const unsigned long long hit = __ballot(t > 0 && lo <= a && a < before + incl);
            if (hit) {
                const int L = __ffsll(hit) - 1;
                cs = base + L;
                cs_n = __builtin_amdgcn_readlane(n, L);
                seq_base = before + __builtin_amdgcn_readlane(incl - t, L);
                break;
            }
            before += __builtin_amdgcn_readlane(incl, kWave - 1);
        }
    }

    // A position in the tile stream: segment (s, g) of nb tiles (np units)
    // whose first unit has index seg; block bi counted from the sequence's
    // first streamed block pre (0 unless it is in a prefix group), n the
    // length counted from there; the current piece of the segment ends at
    // block hi (the slice's end, the segment's end, or with PART the
    // partition's end). All fields are wave-uniform.
    struct Cursor {
        int s, g, n, pre, nb, np, bi, hi;
        int64_t seg;
    };
    // Move c, which has just reached the end of its piece (bi == hi), to the
    // first block of the next piece inside the slice: the next partition of
    // the segment (PART), else the first block of the next segment (order s,
    // then g). false when the slice has no more tiles.
    auto next_piece = [&](Cursor& c) -> bool {
        if constexpr (PART) {
            if (c.bi < c.nb) {
                if (c.seg + c.bi / pt >= b) return false;
                c.hi = min(c.nb, c.bi + pt);
                return true;
            }
        }
        const int64_t seg = c.seg + c.np;
        if (seg >= b) return false;
        if (c.g + 1 < H) {
            ++c.g;
        } else {
            int s = c.s + 1, n = 0, pre = 0, nb = 0;
            for (; s < S; ++s) {
                n = len_uniform(s);
                pre = pre_uniform(s);
                nb = tiles_of(n, pre, max_ctx);
                if (nb > 0) break;
            }
            if (s >= S) return false;  // cannot happen: tiles after seg exist
            c.s = s;
            c.g = 0;
            c.n = n - pre * kBlock;
            c.pre = pre;
            c.nb = nb;
            c.np = units_of(nb);
        }
        c.seg = seg;
        c.bi = 0;
        c.hi = PART ? min(c.nb, pt) : (int)min((int64_t)c.nb, b - seg);
        return true;
    };

    Cursor cc;  // the tile being computed
    cc.s = cs;
    cc.pre = pre_uniform(cs);
    cc.n = cs_n;
    cc.nb = tiles_of(cc.n, cc.pre, max_ctx);
    cc.n -= cc.pre * kBlock;
    if (cc.nb == 0) return;  // cannot happen: unit a lies in a non-empty sequence
    cc.np = units_of(cc.nb);
    cc.g = (int)((a - seq_base) / cc.np);
    cc.seg = seq_base + (int64_t)cc.g * cc.np;
    if constexpr (PART) {
        cc.bi = (int)(a - cc.seg) * pt;
        cc.hi = min(cc.nb, cc.bi + pt);
    } else {
        cc.bi = (int)(a - cc.seg);
        cc.hi = (int)min((int64_t)cc.nb, cc.bi + (b - a));
    }
    int clo = cc.bi;           // first block of the computed piece
    bool first_piece = true;   // the piece holding unit a (partial slot 0)
    bool piece_bad = false;

    Cursor ic = cc;  // the next tile to load (kPrefetch tiles ahead of cc)
    bool ic_valid = true;
    // Block id of ic's tile, read one tile before it is needed; -1 marks an
    // id outside the pool.
    auto read_id = [&](const Cursor& c) -> int {
        const int id = uniform_read(p.block_tables, (size_t)c.s * mb + c.pre + c.bi);
        return (id < 0 || id >= p.num_blocks) ? -1 : id;
    };
    int ic_id = read_id(ic);
    auto ic_advance = [&]() {
        if (!ic_valid) return;
        if (++ic.bi == ic.hi) ic_valid = next_piece(ic);
        if (ic_valid) ic_id = read_id(ic);
    };

    // Lane roles in the MFMA layouts: column t = l % 16 (the head for scores,
    // the token for K operands, the element for V operands and outputs) and
    // k-group g4 = l / 16.
    const int t = lane & 15;
    const int g4 = lane >> 4;
    const uint32_t k_off = (uint32_t)((g4 * kBlock + t) * 8 * KB);  // slab g4, token t
    const uint32_t v_off = (uint32_t)((t * 4 + g4) * 8 * KB);  // column t, tokens 4*g4..
    const int x16 = (lane ^ 16) << 2, x32 = (lane ^ 32) << 2;       // cross-group partners
    int head_lane[4];                                                // lane holding head 4*g4 + j
#pragma unroll
    for (int j = 0; j < 4; ++j) head_lane[j] = (4 * g4 + j) << 2;

    // q: the query of the piece being computed; q_nx: that of the next
    // segment, read as soon as the tile stream reaches it.
    typename TM::Q q, q_nx;
    auto load_q = [&](typename TM::Q& dst, int s, int g) {
        TM::load_q(dst, p.q + ((size_t)s * Hq + (size_t)g * G + t) * D * QB, t < G, g4);
    };

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
        return TileRef{tile_elem_offset(ic_id, ic.g, H, D) * KB, kTileBytes};
    };
    uint32_t kr[kPrefetch][NK][KW], vr[kPrefetch][NVL][VLW];
    bool slot_bad[kPrefetch];
    // Each tile is read through its own buffer resource (base = the tile),
    // nontemporal: every cache byte is used once per call. The scheduling
    // barriers keep the loads of a refill together.
    auto issue_k = [&](int slot, TileRef t_) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(p.k_cache + t_.off, t_.bytes);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NK; ++i) load_dwords<KW>(r, k_off + i * 4 * kBlock * 8 * KB, kr[slot][i]);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto issue_v = [&](int slot, TileRef t_) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(p.v_cache + t_.off, t_.bytes);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NVL; ++i) load_dwords<VLW>(r, v_off + i * 32 * kBlock * KB, vr[slot][i]);
        __builtin_amdgcn_sched_barrier(0);
    };

    // The query first: the oldest load in flight, so the first tile's wait
    // covers it and the loop never has to wait for everything.
    load_q(q, cc.s, cc.g);
#pragma unroll
    for (int slot = 0; slot < kPrefetch; ++slot) {
        const TileRef tr = ic_tile(slot_bad[slot]);
        issue_k(slot, tr);
        issue_v(slot, tr);
        ic_advance();
    }

    // Running state of the piece: max m and weight sum l of head t (this
    // lane's share of the tokens), accumulators of heads 4*g4 + r.
    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t o[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const float qk_scale = p.qk_scale_log2;
    bool active = true;  // cc holds a tile still to compute

    // Balanced split: split segments whose partials this wave was the last to
    // deliver. Only the first and the last piece of a slice can be partial,
    // so there are at most two; they are merged after the stream, which keeps
    // the merge's loads and registers out of the streaming loop. (Fixed
    // partitions are merged by a second launch.)
    struct Pending {
        int s, g, pre, nb;
        int64_t seg;
    };
    Pending pend0{}, pend1{};
    int npend = 0;

    // Every pass of the loop computes one tile per ring slot and issues the
    // loads that refill the slot, unconditionally: a pass after the last
    // tile only reads zeros and computes on data nobody keeps. Only the piece
    // bookkeeping depends on `active`.
    while (active) {
#pragma unroll
        for (int slot = 0; slot < kPrefetch; ++slot) {
            piece_bad |= slot_bad[slot];
            bool next_bad;
            const TileRef nxt = ic_tile(next_bad);
            // The tile about to be loaded opens the next segment (with one
            // tile in flight, the current tile then ends this piece): its
            // query is read first, so the in-order wait for that tile covers
            // it too and the piece change waits for nothing else.
            static_assert(kPrefetch == 1, "the next segment's query is read one tile ahead");
            if (ic_valid && ic.seg != cc.seg) load_q(q_nx, ic.s, ic.g);

            // ---- scores; the next K goes out as soon as this K is consumed ----
            f32x4_t sc = TM::qk(kr[slot], q);
            settle(sc);
            issue_k(slot, nxt);

            float x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = sc[j] * qk_scale;
            const int live = cc.n - cc.bi * kBlock;  // tokens < live hold positions < n
            if (live < kBlock) {
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = 4 * g4 + j < live ? x[j] : -INFINITY;
                TM::mask_v(vr[slot], live - 4 * g4);
            }

            // ---- online softmax: move the max only when a score outgrows it ----
            const float xm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            if (__any(xm > m_run + kLazyRescale)) {
                float tm = fmaxf(xm, lane_fetch(x16, xm));
                tm = fmaxf(tm, lane_fetch(x32, tm));  // tile max of head t
                const float mn = fmaxf(m_run, tm);
                const float c = __builtin_amdgcn_exp2f(m_run - mn);
                l_run *= c;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float cr = lane_fetch(head_lane[r], c);  // factor of head 4*g4 + r
#pragma unroll
                    for (int j = 0; j < NV; ++j) o[j][r] *= cr;
                }
                m_run = mn;
            }
            float pr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) pr[j] = __builtin_amdgcn_exp2f(x[j] - m_run);

            // ---- P.V; the next V goes out once this V is consumed ----
            l_run += TM::pv(pr, vr[slot], o);
#pragma unroll
            for (int j = 0; j < NV; ++j) settle(o[j]);
            issue_v(slot, nxt);
            slot_bad[slot] = next_bad;
            ic_advance();

            if (!active) continue;
            if (++cc.bi < cc.hi) continue;

            // ---- the piece [clo, hi) is done: write it out, or leave a partial ----
            float lt = l_run + lane_fetch(x16, l_run);
            lt += lane_fetch(x32, lt);  // weight sum of head t over the piece
            const size_t orow = (size_t)cc.s * Hq + (size_t)cc.g * G;  // first output row
            if (PFX && cc.pre > 0 && clo == 0 && cc.hi == cc.nb) {
                // the whole suffix of a grouped sequence: float32 result
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int hh = 4 * g4 + r;
                    const float inv = 1.f / lane_fetch(head_lane[r], lt);
                    if (hh < G) {
#pragma unroll
                        for (int j = 0; j < NV; ++j)
                            p.res_o[(orow + hh) * D + 16 * j + t] = piece_bad ? nan : o[j][r] * inv;
                    }
                }
                if (lane < G) p.res_lse[orow + lane] = piece_bad ? nan : m_run + __log2f(lt);
            } else if (clo == 0 && cc.hi == cc.nb) {
                // the whole segment: normalise and store
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int hh = 4 * g4 + r;
                    const float sc_r = p.v_scale / lane_fetch(head_lane[r], lt);
                    if (hh < G) {
#pragma unroll
                        for (int j = 0; j < NV; ++j)
                            store_f32_as<QT>(p.out, (orow + hh) * D + 16 * j + t,
                                             piece_bad ? nan : o[j][r] * sc_r);
                    }
                }
            } else if constexpr (PART) {
                // partition j of a split segment: unnormalised accumulator,
                // max, sum to its own slot, plain nontemporal stores; the
                // merge launch that follows (the kernel boundary orders them)
                // reduces them. (The stores hold up the in-order wait for the
                // next tiles until they complete; nontemporal ones complete
                // sooner: 220 -> 215 us for 16 x 32768 fp8 in 512-token
                // partitions.)
                float* slotp = p.slots +
                               ((size_t)(cc.s * H + cc.g) * p.part_stride + clo / pt) * SLOT;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int hh = 4 * g4 + r;
                    if (hh < GM) {
#pragma unroll
                        for (int j = 0; j < NV; ++j)
                            __builtin_nontemporal_store(o[j][r], slotp + hh * D + 16 * j + t);
                    }
                }
                if (lane < GM) {
                    __builtin_nontemporal_store(piece_bad ? nan : m_run, slotp + GM * D + lane);
                    __builtin_nontemporal_store(piece_bad ? nan : lt, slotp + GM * D + GM + lane);
                }
            } else {
                // partial of a split segment: unnormalised accumulator, max, sum
                float* slotp = p.slots + (size_t)(2 * w + (first_piece ? 0 : 1)) * SLOT;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int hh = 4 * g4 + r;
                    if (hh < GM) {
#pragma unroll
                        for (int j = 0; j < NV; ++j) coherent_store(slotp + hh * D + 16 * j + t, o[j][r]);
                    }
                }
                if (lane < GM) {
                    coherent_store(slotp + GM * D + lane, piece_bad ? nan : m_run);
                    coherent_store(slotp + GM * D + GM + lane, piece_bad ? nan : lt);
                }
                // The partial has landed before it is announced: wait for the
                // write-through stores to complete, and keep the compiler from
                // moving any memory access across the wait and the counter.
                __builtin_amdgcn_s_waitcnt(0);
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                int* counter = p.counters + (size_t)cc.s * H + cc.g;
                int old = 0;
                if (lane == 0)
                    old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                old = __builtin_amdgcn_readfirstlane(old);
                // No load of the partials may be hoisted above the counter read.
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                const int w0 = worker_of(cc.seg, total, nw);
                const int w1 = worker_of(cc.seg + cc.nb - 1, total, nw);
                if (old == w1 - w0) {  // every partial of the segment is in
                    const Pending pd{cc.s, cc.g, cc.pre, cc.nb, cc.seg};
                    if (npend == 0) pend0 = pd; else pend1 = pd;
                    ++npend;
                }
            }

            // ---- next piece (its first tiles are already in flight) ----
            const bool same_segment = PART && cc.bi < cc.nb;
            if (!next_piece(cc)) {
                active = false;
                continue;
            }
            clo = cc.bi;
            first_piece = false;
            piece_bad = false;
            if (!same_segment) q = q_nx;  // read with the segment's first tile, before it
            m_run = -INFINITY;
            l_run = 0.f;
#pragma unroll
            for (int j = 0; j < NV; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }

    // Merge the split segments this wave completed (log-sum-exp over the
    // partials) and leave their counters at zero for the next call.
    for (int i = 0; i < npend; ++i) {
        const Pending& pd = i == 0 ? pend0 : pend1;
        const int w0 = worker_of(pd.seg, total, nw);
        const int w1 = worker_of(pd.seg + pd.nb - 1, total, nw);
        const int k0 = (int64_t)w0 * total / nw < pd.seg ? 1 : 0;
        // worker w0's partial is in its slot k0, the others' in their slot 0
        merge_segment<QT, D, GM>(
            p, w1 - w0 + 1,
            [&](int j) { return p.slots + (size_t)(2 * (w0 + j) + (j == 0 ? k0 : 0)) * SLOT; }, G,
            (size_t)pd.s * Hq + (size_t)pd.g * G, lane, PFX && pd.pre > 0);
        if (lane == 0)
            __hip_atomic_store(p.counters + (size_t)pd.s * H + pd.g, 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Worker waves per CU a default decode launch aims at: about 12 KiB of K
// tiles (and as much V) in flight per CU with one tile per wave, i.e. 3 for
// 16-bit d 128 tiles and 6 for fp8 d 128, clamped to 2..8. Measured on the
// 40 x 8192 fp16 GQA shape, 3 per CU is best (a sweep over 2..16 per CU):
// more concurrent streams lower the bandwidth the memory system delivers
// and widen the spread between waves. fp8 tiles carry half the bytes, and
// the 16 x 32768 fp8 shape runs 27% faster at 6 per CU than at 3. The suffix
// pass of the shared-prefix call (short segments, the prefix pass running
// beside it) takes one more: 256 sequences with 64..512-token suffixes,
// 96.0 us per call at 4 per CU against 98.6 at 3 (2, 5, 6 and 8 per CU were
// slower).
template <int KT, int D, bool PFX>
constexpr int decode_waves_per_cu() {
    constexpr int kTileBytes = kBlock * D * Elem<KT>::bytes;
    constexpr int kTarget = 12288 / kTileBytes < 2 ? 2 : 12288 / kTileBytes > 8 ? 8 : 12288 / kTileBytes;
    return PFX ? (kTarget + 1 > 8 ? 8 : kTarget + 1) : kTarget;
}

// Compute units of the current device (0 if it cannot be read), cached per
// device.
int device_cus();

// The decode launch's parameters for a call with nw worker waves (pt: tiles
// per fixed partition, 1 for the balanced split).
template <int KT>
inline DecodeParams decode_params(const DecodeArgs& a, int nw, int pt, bool part, bool pfx) {
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
    p.part_tiles = pt;
    p.part_stride = part ? (a.max_blocks_per_seq + pt - 1) / pt : 0;
    p.qk_scale_log2 = a.scale * (KT == PKV_FP8_E4M3 ? a.k_scale : 1.f) * kLog2e;
    p.v_scale = KT == PKV_FP8_E4M3 ? a.v_scale : 1.f;
    p.counters = a.counters;
    p.slots = a.slots;
    p.out = a.out;
    p.num_groups = pfx ? a.num_groups : 0;
    p.group_starts = a.group_starts;
    p.group_prefix = a.group_prefix;
    p.res_o = a.res_o;
    p.res_lse = a.res_lse;
    return p;
}

}  // namespace pkv
