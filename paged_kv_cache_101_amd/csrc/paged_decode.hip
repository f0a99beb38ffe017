// paged_decode.hip -- paged decode attention for gfx950 (CDNA4), one launch.
//
// The per-wave work (what is computed, the split, the tile math, the merge)
// is decode_wave() in decode_wave.h; this file holds the decode kernel that
// runs one worker wave per workgroup, the fixed-partition reduce and the
// host launch code.
#include <atomic>

#include "decode_wave.h"

namespace pkv {

template <int KT, int QT, int D, int GM, bool PFX, bool PART>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void paged_decode_kernel(DecodeParams p) {
    decode_wave<KT, QT, D, GM, PFX, PART>(
        p, __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kWavesPerGroup) + wave_id()));
}

// ---- fixed partitions: the cross-partition reduce --------------------------------
//
// After a fixed-partition decode launch, every (sequence, KV head) segment
// with more than one partition has left partition j's unnormalised
// accumulator acc_j, maximum m_j and sum l_j (log2 units) in slot j of its
// workspace row. One wave per (sequence, query head) row reduces them by the
// log-sum-exp rule,
//   M = max_j m_j,  out = v_scale * sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j,
// reading them with plain loads (the kernel boundary orders them after the
// decode launch). Rows of segments with one partition were written by the
// decode launch itself and are skipped, as are rows of sequences without
// tiles; a NaN partial (a block id outside the pool) makes the row NaN.
struct PartitionMergeParams {
    const int32_t* context_lens;
    const float* slots;  // [S][H_kv][part_stride][SLOT]
    void* out;
    int num_seqs, num_q_heads, num_kv_heads, group, max_blocks_per_seq;
    int part_tiles, part_stride;
    float v_scale;
};

constexpr int kMergeWaves = 4;  // rows per workgroup of the reduce

template <int QT, int D, int GM>
__global__ __launch_bounds__(kMergeWaves * kWave) void partition_merge_kernel(PartitionMergeParams p) {
    constexpr int SLOT = decode_slot_floats(GM, D);
    constexpr int EPL = D / kWave;  // output elements per lane
    static_assert(D % kWave == 0, "head size must be a multiple of the wave width");
    const int lane = lane_id();
    const int row = (int)blockIdx.x * kMergeWaves + wave_id();
    if (row >= p.num_seqs * p.num_q_heads) return;
    const int s = row / p.num_q_heads, h = row % p.num_q_heads;
    const int g = h / p.group, hh = h % p.group;
    const int nb = tiles_of(p.context_lens[s], 0, p.max_blocks_per_seq * kBlock);
    const int np = (nb + p.part_tiles - 1) / p.part_tiles;
    if (np <= 1) return;
    const float* base = p.slots + (size_t)(s * p.num_kv_heads + g) * p.part_stride * SLOT;
    // Lane j holds partition j0 + j's maximum and sum (partitions 64 at a
    // time; lanes past the last re-read it and drop it), so the weights cost
    // one memory round; the accumulators then follow with 16 partitions'
    // loads in flight, each weight taken from its lane. (Reading each
    // partition's maximum and sum in the accumulator loop, 8 partitions in
    // flight, cost about 3 us more per call for 16 x 32768 tokens at 64
    // query heads; 32 in flight was no faster than 16.)
    float M = -INFINITY;
    if (np > kWave) {
        for (int j0 = 0; j0 < np; j0 += kWave) {
            const float m = base[(size_t)min(j0 + lane, np - 1) * SLOT + GM * D + hh];
            M = fmaxf(M, wave_max(j0 + lane < np ? m : -INFINITY));
        }
    }
    float L = 0.f, acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    for (int j0 = 0; j0 < np; j0 += kWave) {
        const bool live = j0 + lane < np;
        const float* sl = base + (size_t)min(j0 + lane, np - 1) * SLOT;
        const float m = sl[GM * D + hh], l = sl[GM * D + GM + hh];
        if (np <= kWave) M = wave_max(live ? m : -INFINITY);
        const float w = live ? __builtin_amdgcn_exp2f(m - M) : 0.f;
        L += wave_sum(w * l);
        const int cnt = min(kWave, np - j0);
        constexpr int kBatch = 16;
        for (int jb = 0; jb < cnt; jb += kBatch) {
            // a batch of partitions' accumulators, loaded unconditionally
            // (past the last: the last again, with weight zero)
            float a[kBatch][EPL];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const float* sj = base + (size_t)(j0 + min(jb + u, cnt - 1)) * SLOT;
#pragma unroll
                for (int e = 0; e < EPL; ++e) a[u][e] = sj[hh * D + lane * EPL + e];
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const float wu = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), min(jb + u, kWave - 1)));
                const float wj = jb + u < cnt ? wu : 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[e] = fmaf(wj, a[u][e], acc[e]);
            }
        }
    }
    const float sc = p.v_scale / L;
    const size_t orow = (size_t)s * p.num_q_heads + h;
#pragma unroll
    for (int e = 0; e < EPL; ++e) store_f32_as<QT>(p.out, orow * D + lane * EPL + e, acc[e] * sc);
}

// ---- dispatch ------------------------------------------------------------------

// Compute units of the current device, read once per device.
int device_cus() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cus_cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev < 0 || dev >= kMaxDevices) {
        int cus = 0;
        return hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? cus : 0;
    }
    int cus = cus_cache[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cus_cache[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

template <int KT, int QT, int D, int GM, bool PFX, bool PART>
static hipError_t launch_typed(const DecodeArgs& a) {
    auto kernel = paged_decode_kernel<KT, QT, D, GM, PFX, PART>;
    const int pt = PART ? a.partition_size / kBlock : 1;
    // units of work at most: tiles, or partitions of pt tiles (PART)
    const int64_t unit_bound = (int64_t)a.num_seqs * a.num_kv_heads *
                               ((a.max_blocks_per_seq + pt - 1) / pt);
    int nw = a.num_workers;
    if (nw == 0) {
        constexpr int kWant = decode_waves_per_cu<KT, D, PFX>();
        // occupancy of this kernel (the same on every device of this kind)
        static std::atomic<int> per_cu_cache{0};
        int per_cu = per_cu_cache.load(std::memory_order_relaxed);
        if (per_cu == 0) {
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) !=
                    hipSuccess ||
                per_cu <= 0)
                per_cu = 1;
            per_cu_cache.store(per_cu, std::memory_order_relaxed);
        }
        const int cus = device_cus();
        if (cus <= 0) return hipErrorInvalidDevice;
        nw = (per_cu < kWant ? per_cu : kWant) * cus * kWavesPerGroup;
        if (nw > kMaxWorkers) nw = kMaxWorkers;
        if (PART) {
            // whole partitions per wave: the nearest whole number k of them
            // for the full batch, and as many waves as that needs
            int64_t k = (unit_bound + nw / 2) / nw;
            if (k < 1) k = 1;
            const int64_t want = (unit_bound + k - 1) / k;
            nw = (int)(want < kMaxWorkers ? want : kMaxWorkers);
        }
    }
    // never more workers than units could exist
    if (nw > unit_bound) nw = (int)unit_bound;
    if (nw < 1) nw = 1;

    const DecodeParams p = decode_params<KT>(a, nw, pt, PART, PFX);
    const int grid = (nw + kWavesPerGroup - 1) / kWavesPerGroup;
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, a.stream, p);
    if constexpr (PART) {
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        PartitionMergeParams mp;
        mp.context_lens = a.context_lens;
        mp.slots = a.slots;
        mp.out = a.out;
        mp.num_seqs = a.num_seqs;
        mp.num_q_heads = a.num_q_heads;
        mp.num_kv_heads = a.num_kv_heads;
        mp.group = a.group;
        mp.max_blocks_per_seq = a.max_blocks_per_seq;
        mp.part_tiles = p.part_tiles;
        mp.part_stride = p.part_stride;
        mp.v_scale = p.v_scale;
        const int64_t rows = (int64_t)a.num_seqs * a.num_q_heads;
        hipLaunchKernelGGL((partition_merge_kernel<QT, D, GM>),
                           dim3((unsigned)((rows + kMergeWaves - 1) / kMergeWaves)),
                           dim3(kMergeWaves * kWave), 0, a.stream, mp);
    }
    return hipGetLastError();
}

template <int KT, int QT, int D, bool PFX, bool PART>
static hipError_t launch_group(const DecodeArgs& a) {
    switch (padded_group(a.group)) {
    case 1: return launch_typed<KT, QT, D, 1, PFX, PART>(a);
    case 2: return launch_typed<KT, QT, D, 2, PFX, PART>(a);
    case 4: return launch_typed<KT, QT, D, 4, PFX, PART>(a);
    case 6: return launch_typed<KT, QT, D, 6, PFX, PART>(a);
    default: return launch_typed<KT, QT, D, 8, PFX, PART>(a);
    }
}

template <int KT, int QT, int D>
static hipError_t launch_mode(const DecodeArgs& a) {
    if (a.res_o != nullptr) return launch_group<KT, QT, D, true, false>(a);  // suffix pass
    if (a.partition_size > 0) return launch_group<KT, QT, D, false, true>(a);
    return launch_group<KT, QT, D, false, false>(a);
}

template <int KT, int QT>
static hipError_t launch_dim(const DecodeArgs& a) {
    return a.head_dim == 64 ? launch_mode<KT, QT, 64>(a) : launch_mode<KT, QT, 128>(a);
}

hipError_t launch_paged_decode(const DecodeArgs& a) {
    if (a.kv_dtype == PKV_F32) return launch_dim<PKV_F32, PKV_F32>(a);
    if (a.kv_dtype == PKV_F16) return launch_dim<PKV_F16, PKV_F16>(a);
    if (a.kv_dtype == PKV_BF16) return launch_dim<PKV_BF16, PKV_BF16>(a);
    if (a.q_dtype == PKV_F16) return launch_dim<PKV_FP8_E4M3, PKV_F16>(a);
    return launch_dim<PKV_FP8_E4M3, PKV_BF16>(a);
}

}  // namespace pkv
