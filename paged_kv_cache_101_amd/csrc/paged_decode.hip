// paged_decode.hip -- paged decode attention for gfx950 (CDNA4), one launch.
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
constexpr int kWavesPerGroup = 1;  // one worker wave per workgroup: any count spreads evenly
constexpr int kThreads = kWavesPerGroup * kWave;
constexpr int kPrefetch = 1;  // tiles whose K and V a wave has in flight

// Scores are kept in log2 units; a wave only rescales its running sums when a
// new score exceeds its running max by more than kLazyRescale (2^8 headroom
// for the unnormalised weights, far inside float32 and f16 range). The result
// is the same softmax: every weight is exp2(x - m) against one common m.
constexpr float kLazyRescale = 8.0f;

typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// N dwords at byte `voff` of a buffer resource, nontemporal.
template <int N>
__device__ __forceinline__ void load_dwords(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t* w) {
    constexpr int kNontemporal = 2;
    if constexpr (N == 1) {
        w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, kNontemporal);
    } else if constexpr (N == 2) {
        const u32x2_t a = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, kNontemporal);
        w[0] = a[0];
        w[1] = a[1];
    } else {
        static_assert(N % 4 == 0, "dword count");
#pragma unroll
        for (int c = 0; c < N / 4; ++c) {
            const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16 * c, 0, kNontemporal);
#pragma unroll
            for (int i = 0; i < 4; ++i) w[4 * c + i] = a[i];
        }
    }
}

// The per-tile matrix work for cache type KT and query type QT.
//   K: NK loads per lane, load i = the 8-element slab (l/16) + 4i of token l%16;
//   V: NVL loads per lane, load i = tokens 4*(l/16) .. +3 of element columns
//      16*(2i) + l%16 and 16*(2i+1) + l%16 (one 8-element run of the tile).
template <int KT, int QT, int D>
struct TileMath {
    static constexpr int KB = Elem<KT>::bytes;
    static constexpr int QB = Elem<QT>::bytes;
    static constexpr int NK = D / 32;
    static constexpr int NV = D / 16;   // P.V blocks of 16 element columns
    static constexpr int NVL = D / 32;  // V loads (two blocks each)
    static constexpr int KW = 2 * KB;   // dwords per K load (8 elements)
    static constexpr int VW = KB;       // dwords of one block's 4 tokens
    static constexpr int VLW = 2 * VW;  // dwords per V load (8 elements)
    static constexpr bool kF32 = (KT == PKV_F32);
    static constexpr int QW = 8 * QB / 4;  // dwords per query slab

    // Query slabs of head l % 16 matching the K loads (zero for padded heads).
    struct Q {
        uint32_t w[NK][QW];
    };

    __device__ static void load_q(Q& q, const uint8_t* row, bool valid, int g4) {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            if (valid) {
                const uint4* src = reinterpret_cast<const uint4*>(row + (size_t)8 * (g4 + 4 * i) * QB);
#pragma unroll
                for (int c = 0; c < QW / 4; ++c) {
                    const uint4 a = src[c];
                    q.w[i][4 * c] = a.x;
                    q.w[i][4 * c + 1] = a.y;
                    q.w[i][4 * c + 2] = a.z;
                    q.w[i][4 * c + 3] = a.w;
                }
            } else {
#pragma unroll
                for (int c = 0; c < QW; ++c) q.w[i][c] = 0u;
            }
        }
    }

    // Two fp8 codes (bytes 0-1, or 2-3 with `hi`) as two elements of the 16-bit
    // compute type, packed in one dword. Exact: every E4M3 value is an f16
    // and a bf16 value (the scaled conversion runs with scale 1).
    template <bool HI>
    __device__ static uint32_t widen_fp8_pair(uint32_t w) {
        if constexpr (QT == PKV_F16)
            return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
        else
            return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
    }

    // 8 K elements (one slab entry) in the 16-bit compute type.
    template <typename V8>
    __device__ static V8 k_operand(const uint32_t* kw) {
        if constexpr (KT == PKV_FP8_E4M3) {
            u32x4_t u;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                u[2 * i] = widen_fp8_pair<false>(kw[i]);
                u[2 * i + 1] = widen_fp8_pair<true>(kw[i]);
            }
            return __builtin_bit_cast(V8, u);
        } else {
            const u32x4_t u = {kw[0], kw[1], kw[2], kw[3]};
            return __builtin_bit_cast(V8, u);
        }
    }

    // S^T (tokens 4*(l/16) + j, head l % 16) of one tile.
    __device__ static f32x4_t qk(const uint32_t (&kr)[NK][KW], const Q& q) {
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            if constexpr (kF32) {
                // k index of MFMA e is element 8*(l/16 + 4i) + e of token / head
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    s = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, kr[i][e]),
                                                             __builtin_bit_cast(float, q.w[i][e]),
                                                             s, 0, 0, 0);
            } else if constexpr (QT == PKV_F16) {
                const u32x4_t qu = {q.w[i][0], q.w[i][1], q.w[i][2], q.w[i][3]};
                s = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<f16x8_t>(kr[i]),
                                                           __builtin_bit_cast(f16x8_t, qu), s, 0, 0,
                                                           0);
            } else {
                const u32x4_t qu = {q.w[i][0], q.w[i][1], q.w[i][2], q.w[i][3]};
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<bf16x8_t>(kr[i]),
                                                            __builtin_bit_cast(bf16x8_t, qu), s, 0,
                                                            0, 0);
            }
        }
        return s;
    }

    // Zero the V elements of tokens this lane holds at or past the live count
    // (nlive = live tokens among its four, any integer).
    __device__ static void mask_v(uint32_t (&vr)[NVL][VLW], int nlive) {
        uint32_t m[VW];
        if constexpr (VW == 1) {
            m[0] = nlive >= 4 ? ~0u : nlive <= 0 ? 0u : (1u << (8 * nlive)) - 1u;
        } else if constexpr (VW == 2) {
            m[0] = nlive >= 2 ? ~0u : nlive == 1 ? 0xFFFFu : 0u;
            m[1] = nlive >= 4 ? ~0u : nlive == 3 ? 0xFFFFu : 0u;
        } else {
#pragma unroll
            for (int i = 0; i < VW; ++i) m[i] = i < nlive ? ~0u : 0u;
        }
#pragma unroll
        for (int j = 0; j < NVL; ++j)
#pragma unroll
            for (int i = 0; i < VLW; ++i) vr[j][i] &= m[i % VW];
    }

    // o[j] (heads 4*(l/16) + r, element 16j + l%16) += P . V_tile; returns the
    // sum of this lane's four weights as they entered the product.
    // (block j's 4 tokens: dwords (j % 2) * VW .. of load j / 2)
    __device__ static float pv(const float (&pr)[4], const uint32_t (&vr)[NVL][VLW], f32x4_t (&o)[NV]) {
        if constexpr (kF32) {
#pragma unroll
            for (int j = 0; j < NV; ++j)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    o[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        pr[kk], __builtin_bit_cast(float, vr[j / 2][(j % 2) * VW + kk]), o[j], 0, 0, 0);
            return (pr[0] + pr[1]) + (pr[2] + pr[3]);
        } else if constexpr (QT == PKV_F16) {
            const f16x4_t a = {(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3]};
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                f16x4_t b;
                const uint32_t* vj = &vr[j / 2][(j % 2) * VW];
                if constexpr (KT == PKV_FP8_E4M3) {
                    const u32x2_t u = {widen_fp8_pair<false>(vj[0]), widen_fp8_pair<true>(vj[0])};
                    b = __builtin_bit_cast(f16x4_t, u);
                } else {
                    const u32x2_t u = {vj[0], vj[1]};
                    b = __builtin_bit_cast(f16x4_t, u);
                }
                o[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, o[j], 0, 0, 0);
            }
            return ((float)a[0] + (float)a[1]) + ((float)a[2] + (float)a[3]);
        } else {
            const bf16x4_t a = {(__bf16)pr[0], (__bf16)pr[1], (__bf16)pr[2], (__bf16)pr[3]};
            const i16x4_t ai = __builtin_bit_cast(i16x4_t, a);
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                i16x4_t b;
                const uint32_t* vj = &vr[j / 2][(j % 2) * VW];
                if constexpr (KT == PKV_FP8_E4M3) {
                    const u32x2_t u = {widen_fp8_pair<false>(vj[0]), widen_fp8_pair<true>(vj[0])};
                    b = __builtin_bit_cast(i16x4_t, u);
                } else {
                    const u32x2_t u = {vj[0], vj[1]};
                    b = __builtin_bit_cast(i16x4_t, u);
                }
                o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ai, b, o[j], 0, 0, 0);
            }
            return ((float)a[0] + (float)a[1]) + ((float)a[2] + (float)a[3]);
        }
    }
};

// Value of `v` in lane addr / 4 (addr a byte address, as the LDS crossbar
// takes it; no LDS memory is used).
__device__ __forceinline__ float lane_fetch(int addr, float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(addr, __builtin_bit_cast(int, v)));
}

// Everything that computes v happens before this point, and no memory access
// moves across it. Placed between the last use of a ring slot and the loads
// that refill it, it keeps the compiler from sinking that use past the refill
// (which would make the slot's old and new contents live at once, land the
// refill in other registers and copy it back at the loop latch).
__device__ __forceinline__ void settle(f32x4_t& v) { asm volatile("" : "+v"(v) : : "memory"); }

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
    using TM = TileMath<KT, QT, D>;
    constexpr int NK = TM::NK, NV = TM::NV, NVL = TM::NVL, KW = TM::KW, VLW = TM::VLW;
    constexpr int KB = Elem<KT>::bytes;
    constexpr int QB = Elem<QT>::bytes;
    constexpr uint32_t kTileBytes = (uint32_t)kBlock * D * KB;
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
    // Block id of ic's tile, read one tile before it is needed; -1 marks an
    // id outside the pool.
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

    typename TM::Q q;
    auto load_q = [&](int s, int g) {
        TM::load_q(q, p.q + ((size_t)s * Hq + (size_t)g * G + t) * D * QB, t < G, g4);
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
    load_q(cc.s, cc.g);
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
    // tile only reads zeros and computes on data nobody keeps. Only the piece
    // bookkeeping depends on `active`.
    while (active) {
#pragma unroll
        for (int slot = 0; slot < kPrefetch; ++slot) {
            piece_bad |= slot_bad[slot];
            bool next_bad;
            const TileRef nxt = ic_tile(next_bad);

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
            if (cc.bi + 1 < cc.hi) {
                ++cc.bi;
                continue;
            }

            // ---- the piece is done: write it out, or leave a partial ----
            float lt = l_run + lane_fetch(x16, l_run);
            lt += lane_fetch(x32, lt);  // weight sum of head t over the piece
            const size_t orow = (size_t)cc.s * Hq + (size_t)cc.g * G;  // first output row
            if (clo == 0 && cc.hi == cc.nb) {
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
        // three worker waves per CU
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
        // three waves per CU: measured best on the 40 x 8192 GQA shape (a sweep
        // over 2..16 per CU); more concurrent streams lower the bandwidth the
        // memory system delivers and widen the spread between waves
        nw = (per_cu < 3 ? per_cu : 3) * cus * kWavesPerGroup;
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
