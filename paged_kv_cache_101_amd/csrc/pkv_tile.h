// pkv_tile.h -- the per-tile attention arithmetic on the matrix cores, and
// the wave-level helpers that the decode kernels share.
//
// One tile is 16 tokens of one KV head (one physical block). Against it, a
// wave holds up to 16 query rows (the G heads of one sequence in decode, or 16
// (sequence, head) rows in the shared-prefix pass) as the columns of the 16x16
// MFMA shapes: lane l serves column l % 16 in k-group l / 16.
#pragma once

#include "pkv_device.h"

namespace pkv {

constexpr float kLog2e = 1.44269504088896340736f;

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

// Cache policies of a buffer load: nontemporal for data read once per call
// (decode's private tiles), the default for data several waves re-read
// (shared-prefix tiles).
constexpr int kLoadNontemporal = 2;
constexpr int kLoadCached = 0;

// N dwords at byte `voff` of a buffer resource.
template <int N, int AUX = kLoadNontemporal>
__device__ __forceinline__ void load_dwords(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t* w) {
    if constexpr (N == 1) {
        w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, AUX);
    } else if constexpr (N == 2) {
        const u32x2_t a = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, AUX);
        w[0] = a[0];
        w[1] = a[1];
    } else {
        static_assert(N % 4 == 0, "dword count");
#pragma unroll
        for (int c = 0; c < N / 4; ++c) {
            const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16 * c, 0, AUX);
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
            // bfloat16 keeps 8 significant bits: with a bfloat16 cache each
            // weight enters as a rounded high part plus the rounded
            // remainder (about 16 bits together), two products per element
            // block, and the output is then the correctly rounded result in
            // all but about 0.2% of elements (about 60% with one part: on
            // two- to four-token contexts single weights move the average).
            // fp8 caches keep one part: their long contexts average the
            // rounding away, and the second product cost them 3%.
            constexpr bool kSplit = (KT == PKV_BF16);
            const bf16x4_t a = {(__bf16)pr[0], (__bf16)pr[1], (__bf16)pr[2], (__bf16)pr[3]};
            bf16x4_t alo = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
            if constexpr (kSplit)
                alo = bf16x4_t{(__bf16)(pr[0] - (float)a[0]), (__bf16)(pr[1] - (float)a[1]),
                               (__bf16)(pr[2] - (float)a[2]), (__bf16)(pr[3] - (float)a[3])};
            const i16x4_t ai = __builtin_bit_cast(i16x4_t, a);
            const i16x4_t ali = __builtin_bit_cast(i16x4_t, alo);
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
                if constexpr (kSplit) o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ali, b, o[j], 0, 0, 0);
            }
            if constexpr (kSplit)
                return (((float)a[0] + (float)alo[0]) + ((float)a[1] + (float)alo[1])) +
                       (((float)a[2] + (float)alo[2]) + ((float)a[3] + (float)alo[3]));
            return ((float)a[0] + (float)a[1]) + ((float)a[2] + (float)a[3]);
        }
    }

    // Two tiles A and B in one P.V: O += P (16 x 32 keys) . V (32 keys x D)
    // as D/16 MFMA 16x16x32 (16-bit types; not for float32 caches). The key
    // order of the contraction is A's keys 4*(l/16) .. +3, then B's: exactly
    // the four scores a lane holds for each tile, and the matching halves of
    // the two tiles' V loads. Returns the sum of this lane's eight weights as
    // they entered the product.
    __device__ static float pv2(const float (&pa)[4], const float (&pb)[4],
                                const uint32_t (&va)[NVL][VLW], const uint32_t (&vb)[NVL][VLW],
                                f32x4_t (&o)[NV]) {
        static_assert(!kF32, "16-bit operands only");
        if constexpr (QT == PKV_F16) {
            const f16x8_t a = {(_Float16)pa[0], (_Float16)pa[1], (_Float16)pa[2], (_Float16)pa[3],
                               (_Float16)pb[0], (_Float16)pb[1], (_Float16)pb[2], (_Float16)pb[3]};
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                o[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, v_operand<f16x8_t>(va, vb, j), o[j],
                                                              0, 0, 0);
            }
            float l = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) l += (float)a[i];
            return l;
        } else {
            const bf16x8_t a = {(__bf16)pa[0], (__bf16)pa[1], (__bf16)pa[2], (__bf16)pa[3],
                                (__bf16)pb[0], (__bf16)pb[1], (__bf16)pb[2], (__bf16)pb[3]};
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, v_operand<bf16x8_t>(va, vb, j),
                                                               o[j], 0, 0, 0);
            }
            float l = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) l += (float)a[i];
            return l;
        }
    }

    // B operand of element block j for pv2: tile A's 4 tokens, then tile B's.
    template <typename V8>
    __device__ static V8 v_operand(const uint32_t (&va)[NVL][VLW], const uint32_t (&vb)[NVL][VLW],
                                   int j) {
        const uint32_t* xa = &va[j / 2][(j % 2) * VW];
        const uint32_t* xb = &vb[j / 2][(j % 2) * VW];
        if constexpr (KT == PKV_FP8_E4M3) {
            const u32x4_t u = {widen_fp8_pair<false>(xa[0]), widen_fp8_pair<true>(xa[0]),
                               widen_fp8_pair<false>(xb[0]), widen_fp8_pair<true>(xb[0])};
            return __builtin_bit_cast(V8, u);
        } else {
            const u32x4_t u = {xa[0], xa[1], xb[0], xb[1]};
            return __builtin_bit_cast(V8, u);
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

// Integer DPP move of v within 16-lane rows (rows outside ROW_MASK, and
// lanes whose source lies outside their row, read 0).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_int(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row into the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 into rows 2 and 3

// Sum over the wave, returned as a wave-uniform (scalar) value: a DPP sum
// within each 16-lane row, then the four rows' sums read into scalars.
__device__ __forceinline__ int wave_sum_int(int v) {
    v += dpp_int<kDppQuadXor1>(v);
    v += dpp_int<kDppQuadXor2>(v);
    v += dpp_int<kDppRowHalfMirror>(v);
    v += dpp_int<kDppRowMirror>(v);
    return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
           (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// Inclusive prefix sum over the lanes: shifts by 1, 2, 4 and 8 inside each
// 16-lane row, then lane 15's sum into row 1 (and lane 47's into row 3) and
// lane 31's into rows 2 and 3. (Checked on the GPU against a host scan.)
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v += dpp_int<kDppRowShr1>(v);
    v += dpp_int<kDppRowShr2>(v);
    v += dpp_int<kDppRowShr4>(v);
    v += dpp_int<kDppRowShr8>(v);
    v += dpp_int<kDppRowBcast15, 0xA>(v);
    v += dpp_int<kDppRowBcast31, 0xC>(v);
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

// ---- shared-prefix groups -------------------------------------------------
//
// Group j is the run of sequences [starts[j], starts[j+1]) whose first
// prefix[j] logical blocks are the same physical blocks (one copy of a common
// prefix, drpranayjha page, "How PagedAttention pages the KV cache"; ttlab
// page, section 4). A description is usable only as a whole: starts
// non-decreasing inside [0, S] and 0 <= prefix[j] <= max_blocks_per_seq.

// ng if the description is usable, else 0 (every wave computes the same).
__device__ __forceinline__ int usable_groups(const int32_t* starts, const int32_t* prefix, int ng,
                                             int num_seqs, int max_blocks, int lane) {
    if (ng <= 0) return 0;
    bool ok = true;
    for (int base = 0; base < ng; base += kWave) {
        const int j = base + lane;
        if (j < ng) {
            const int a = starts[j], b = starts[j + 1], pj = prefix[j];
            ok = ok && a >= 0 && a <= b && b <= num_seqs && pj >= 0 && pj <= max_blocks;
        }
    }
    return __ballot(!ok) == 0 ? ng : 0;
}

// Shared blocks of sequence s (0 outside every group): the last group whose
// start is <= s, by binary search. UNIFORM: s is wave-uniform (scalar loads).
template <bool UNIFORM>
__device__ __forceinline__ int prefix_blocks_of(const int32_t* starts, const int32_t* prefix,
                                                int ng, int s) {
    if (ng == 0) return 0;
    auto rd = [](const int32_t* b, int i) -> int32_t {
        if constexpr (UNIFORM) return uniform_read(b, (size_t)i);
        else return b[i];
    };
    if (s < rd(starts, 0)) return 0;
    int lo = 0, hi = ng;  // starts[lo] <= s; the group sought is in [lo, hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (rd(starts, mid) <= s) lo = mid;
        else hi = mid;
    }
    return s < rd(starts, lo + 1) ? rd(prefix, lo) : 0;
}

}  // namespace pkv
