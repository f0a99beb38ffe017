// paged_decode.hip -- split-KV paged decode attention for gfx950 (CDNA4).
//
// What is computed (ttlab page, sections 2 and 4; drpranayjha page, "How
// PagedAttention pages the KV cache"; tarundecipher page, "Batching does not
// merge the conversations"): one query token per sequence attends over the
// sequence's own K/V rows, found through its block table in a shared pool of
// 16-token physical blocks; a group of G query heads shares one KV head.
//
// Decomposition
//   * One workgroup (4 waves) owns (sequence s, KV head g, partition j): the
//     positions [j*P, min((j+1)*P, n)). It reads each K and V tile of that
//     range once and serves all G query heads of the group from it.
//   * Tiles are 16 rows x D elements, contiguous. A lane owns 8 consecutive
//     elements of a row, so D/8 lanes cover a row and one wave instruction
//     covers 64*8 contiguous elements: every global load is fully coalesced
//     and goes straight to registers (no LDS staging: each byte is used by
//     exactly the lanes that loaded it).
//   * QK: per-lane dot products (dot2 instructions for 16-bit data), then a
//     DPP sum across the D/8 lanes of the row. Scores go to LDS.
//   * Softmax inside the partition is exact (max over the partition's scores,
//     then exp2), so no running rescale is needed.
//   * PV: each lane accumulates p * V for its 8 elements; the rows a wave
//     covered are summed across lanes, then across waves through LDS.
//   * Several partitions: (m_j, l_j, o_j) go to the workspace and
//     lse_reduce_kernel merges them; one partition: the output is written
//     directly.
// Positions >= n inside the last block are excluded by select (score -inf,
// V row zero), never by arithmetic, so garbage or NaN there cannot leak.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

struct DecodeParams {
    const uint8_t* q;
    const uint8_t* k_cache;
    const uint8_t* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    int num_q_heads;
    int num_kv_heads;
    int group;
    int num_blocks;
    int max_blocks_per_seq;
    int partition_size;
    int num_partitions;
    float qk_scale_log2;  // scale * k_scale * log2(e)
    float v_scale;
    float* ws_m;
    float* ws_l;
    float* ws_o;
    void* out;
};

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kWavesPerGroup = 4;
constexpr int kThreads = kWavesPerGroup * kWave;

template <int KT, int D, int GM>
struct DecodeShape {
    static constexpr int kLanesPerRow = D / kElemsPerLane;          // 16 (D=128) or 8 (D=64)
    static constexpr int kRowsPerInst = kWave / kLanesPerRow;        // 4 or 8
    static constexpr int kInstPerTile = kBlock / kRowsPerInst;       // 4 or 2
    static constexpr int kTileBytes = kBlock * D * Elem<KT>::bytes;
    // Tiles a wave holds in registers at once: 32 KiB per wave for up to 4
    // query heads, 16 KiB above that (the accumulators grow with G).
    static constexpr int kBudget = (GM <= 4 ? 32768 : 16384);
    static constexpr int kBlocksPerWave = kBudget / kTileBytes > 0 ? kBudget / kTileBytes : 1;
    static constexpr int kChunkBlocks = kWavesPerGroup * kBlocksPerWave;
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

// float32 query (f32 caches, and 16-bit queries over fp8 caches).
template <int QT, int KT>
struct QRegsF32 {
    float v[8];
    __device__ __forceinline__ void load(const uint8_t* p) {
        Chunk<QT> c = load_chunk<QT>(p);
        chunk_to_f32<QT>(c, v);
    }
    __device__ __forceinline__ void zero() {
        for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    __device__ __forceinline__ float dot(const Chunk<KT>& k) const {
        float f[8];
        chunk_to_f32<KT>(k, f);
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = fmaf(v[i], f[i], acc);
        return acc;
    }
};
template <>
struct QRegs<PKV_F32, PKV_F32> : QRegsF32<PKV_F32, PKV_F32> {};
template <>
struct QRegs<PKV_F16, PKV_FP8_E4M3> : QRegsF32<PKV_F16, PKV_FP8_E4M3> {};
template <>
struct QRegs<PKV_BF16, PKV_FP8_E4M3> : QRegsF32<PKV_BF16, PKV_FP8_E4M3> {};

template <int KT, int QT, int D, int GM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void paged_decode_partition_kernel(DecodeParams p) {
    using S = DecodeShape<KT, D, GM>;
    constexpr int LPR = S::kLanesPerRow;
    constexpr int RPI = S::kRowsPerInst;
    constexpr int NI = S::kInstPerTile;
    constexpr int BPW = S::kBlocksPerWave;
    constexpr int CHB = S::kChunkBlocks;
    constexpr int KB = Elem<KT>::bytes;
    constexpr int QB = Elem<QT>::bytes;
    constexpr int ROW_BYTES = D * KB;

    extern __shared__ float smem[];
    float* s_scores = smem;                                   // [P][GM]
    float* s_acc = smem + (size_t)p.partition_size * GM;      // [waves][GM][D]
    float* s_ml = s_acc + kWavesPerGroup * GM * D;            // m[GM], l[GM]

    const int j = blockIdx.x;
    const int g = blockIdx.y;
    const int s = blockIdx.z;
    const int lane = lane_id();
    const int wave = wave_id();
    const int P = p.partition_size;
    const int Hq = p.num_q_heads;
    const int G = p.group;
    const bool direct = p.num_partitions == 1;

    const int n = p.context_lens[s];
    const int start = j * P;
    const bool bad_len = n > p.max_blocks_per_seq * kBlock;
    if (n <= 0 || bad_len || start >= n) {
        // Nothing to attend to here. Only a single-partition launch owns the
        // output row; with several partitions the reduce writes it.
        if (direct) {
            const float fill = bad_len ? __builtin_nanf("") : 0.f;
            for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
                const int h = idx / D, e = idx % D;
                store_f32_as<QT>(p.out, ((size_t)s * Hq + g * G + h) * D + e, fill);
            }
        }
        return;
    }
    const int n_p = min(P, n - start);                 // positions in this partition
    const int nb = (n_p + kBlock - 1) / kBlock;        // blocks in this partition
    const int lb0 = start / kBlock;                    // first logical block
    const int32_t* bt_row = p.block_tables + (size_t)s * p.max_blocks_per_seq + lb0;

    const int row_in_inst = lane / LPR;                // which of the RPI rows
    const int col = (lane % LPR) * kElemsPerLane;      // first element this lane owns

    // q for the GM heads of this group (heads past G read as zero).
    QRegs<QT, KT> qr[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        if (h < G)
            qr[h].load(p.q + (((size_t)s * Hq + g * G + h) * D + col) * QB);
        else
            qr[h].zero();
    }

    const uint8_t* kbase = p.k_cache + (size_t)(lane / LPR) * ROW_BYTES + col * KB;
    const uint8_t* vbase = p.v_cache + (size_t)(lane / LPR) * ROW_BYTES + col * KB;
    const int nchunks = (nb + CHB - 1) / CHB;
    int bad_block = 0;

    Chunk<KT> reg[BPW][NI];
    int64_t phys[BPW];

    // ---- phase 1: scores ---------------------------------------------------
    for (int c = 0; c < nchunks; ++c) {
        const int b0 = c * CHB + wave * BPW;
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
            const int b = b0 + i;
            int64_t id = 0;
            if (b < nb) {
                id = bt_row[b];
                if (id < 0 || id >= p.num_blocks) {
                    bad_block = 1;
                    id = 0;
                }
            }
            phys[i] = id;
            if (b < nb) {
                const uint8_t* t = kbase + cache_row_offset(id, g, 0, p.num_kv_heads, ROW_BYTES);
#pragma unroll
                for (int r = 0; r < NI; ++r) reg[i][r] = load_chunk<KT>(t + r * RPI * ROW_BYTES);
            }
        }
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
            const int b = b0 + i;
            if (b >= nb) break;
#pragma unroll
            for (int r = 0; r < NI; ++r) {
                float part[GM];
#pragma unroll
                for (int h = 0; h < GM; ++h) part[h] = group_sum<LPR>(qr[h].dot(reg[i][r]));
                const int t = b * kBlock + r * RPI + row_in_inst;
                if (lane % LPR == 0) {
                    const bool live = t < n_p;
#pragma unroll
                    for (int h = 0; h < GM; ++h)
                        s_scores[t * GM + h] = live ? part[h] * p.qk_scale_log2 : -INFINITY;
                }
            }
        }
    }

    // Start streaming the first V chunk while the softmax runs.
    {
        const int b0 = wave * BPW;
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
            const int b = b0 + i;
            if (b < nb) {
                if (nchunks > 1) {
                    int64_t id = bt_row[b];
                    phys[i] = (id < 0 || id >= p.num_blocks) ? 0 : id;
                }
                const uint8_t* t =
                    vbase + cache_row_offset(phys[i], g, 0, p.num_kv_heads, ROW_BYTES);
#pragma unroll
                for (int r = 0; r < NI; ++r) reg[i][r] = load_chunk<KT>(t + r * RPI * ROW_BYTES);
            }
        }
    }

    bad_block = __syncthreads_or(bad_block);

    // ---- phase 2: softmax of each head over the partition -------------------
    const int ntok = nb * kBlock;
    for (int h = wave; h < G; h += kWavesPerGroup) {
        float mx = -INFINITY;
        for (int t = lane; t < ntok; t += kWave) mx = fmaxf(mx, s_scores[t * GM + h]);
        mx = wave_max(mx);
        float sum = 0.f;
        for (int t = lane; t < ntok; t += kWave) {
            const float e = __builtin_amdgcn_exp2f(s_scores[t * GM + h] - mx);
            s_scores[t * GM + h] = e;
            sum += e;
        }
        sum = wave_sum(sum);
        if (lane == 0) {
            s_ml[h] = mx;
            s_ml[GM + h] = sum;
        }
    }
    __syncthreads();

    // ---- phase 3: P . V ------------------------------------------------------
    float acc[GM][kElemsPerLane];
#pragma unroll
    for (int h = 0; h < GM; ++h)
#pragma unroll
        for (int e = 0; e < kElemsPerLane; ++e) acc[h][e] = 0.f;

    for (int c = 0; c < nchunks; ++c) {
        const int b0 = c * CHB + wave * BPW;
        if (c > 0) {
#pragma unroll
            for (int i = 0; i < BPW; ++i) {
                const int b = b0 + i;
                if (b < nb) {
                    int64_t id = bt_row[b];
                    id = (id < 0 || id >= p.num_blocks) ? 0 : id;
                    const uint8_t* t =
                        vbase + cache_row_offset(id, g, 0, p.num_kv_heads, ROW_BYTES);
#pragma unroll
                    for (int r = 0; r < NI; ++r)
                        reg[i][r] = load_chunk<KT>(t + r * RPI * ROW_BYTES);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
            const int b = b0 + i;
            if (b >= nb) break;
            const bool partial = (b + 1) * kBlock > n_p;
#pragma unroll
            for (int r = 0; r < NI; ++r) {
                const int t = b * kBlock + r * RPI + row_in_inst;
                float pr[GM];
#pragma unroll
                for (int h = 0; h < GM; ++h) pr[h] = s_scores[t * GM + h];
                float vf[kElemsPerLane];
                chunk_to_f32<KT>(reg[i][r], vf);
                if (partial) {
                    const bool live = t < n_p;
#pragma unroll
                    for (int e = 0; e < kElemsPerLane; ++e) vf[e] = live ? vf[e] : 0.f;
                }
#pragma unroll
                for (int h = 0; h < GM; ++h)
#pragma unroll
                    for (int e = 0; e < kElemsPerLane; ++e) acc[h][e] = fmaf(pr[h], vf[e], acc[h][e]);
            }
        }
    }

    // Sum the RPI rows of each wave (lanes with equal `col`), then the waves.
#pragma unroll
    for (int h = 0; h < GM; ++h)
#pragma unroll
        for (int e = 0; e < kElemsPerLane; ++e) {
            float v = acc[h][e];
#pragma unroll
            for (int sh = LPR; sh < kWave; sh <<= 1) v += __shfl_xor(v, sh, kWave);
            acc[h][e] = v;
        }
    if (lane < LPR) {
#pragma unroll
        for (int h = 0; h < GM; ++h)
#pragma unroll
            for (int e = 0; e < kElemsPerLane; ++e)
                s_acc[(wave * GM + h) * D + col + e] = acc[h][e];
    }
    __syncthreads();

    const float nan = __builtin_nanf("");
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
        const int h = idx / D, e = idx % D;
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < kWavesPerGroup; ++w) o += s_acc[(w * GM + h) * D + e];
        const float l = s_ml[GM + h];
        o = bad_block ? nan : o * (p.v_scale / l);
        const size_t row = (size_t)s * Hq + g * G + h;
        if (direct) {
            store_f32_as<QT>(p.out, row * D + e, o);
        } else {
            p.ws_o[(row * p.num_partitions + j) * D + e] = o;
            if (e == 0) {
                p.ws_m[row * p.num_partitions + j] = bad_block ? nan : s_ml[h] * kLn2;
                p.ws_l[row * p.num_partitions + j] = bad_block ? nan : l;
            }
        }
    }
}

// Merge the partitions of one (sequence, query head):
//   M = max_j m_j,  w_j = l_j * exp(m_j - M),  out = sum_j w_j o_j / sum_j w_j
// over the partitions that hold positions (j * P < n).
template <int OT>
__global__ __launch_bounds__(128) void lse_reduce_kernel(
    const float* __restrict__ ws_m, const float* __restrict__ ws_l,
    const float* __restrict__ ws_o, const int32_t* __restrict__ context_lens, int num_q_heads,
    int head_dim, int num_partitions, int partition_size, int max_ctx, void* __restrict__ out) {
    constexpr int kChunk = 512;
    __shared__ float s_w[kChunk];
    __shared__ float s_red[2];
    const int h = blockIdx.x;
    const int s = blockIdx.y;
    const int tid = threadIdx.x;
    const size_t row = (size_t)s * num_q_heads + h;
    const int n = context_lens[s];
    if (n <= 0 || n > max_ctx) {
        const float fill = n <= 0 ? 0.f : __builtin_nanf("");
        for (int e = tid; e < head_dim; e += blockDim.x) store_f32_as<OT>(out, row * head_dim + e, fill);
        return;
    }
    const int pv = (n + partition_size - 1) / partition_size;
    const float* m = ws_m + row * num_partitions;
    const float* l = ws_l + row * num_partitions;
    const float* o = ws_o + row * num_partitions * head_dim;

    float mx = -INFINITY;
    for (int jj = tid; jj < pv; jj += blockDim.x) mx = fmaxf(mx, m[jj]);
    mx = wave_max(mx);
    if ((tid & (kWave - 1)) == 0) s_red[tid / kWave] = mx;
    __syncthreads();
    mx = blockDim.x > kWave ? fmaxf(s_red[0], s_red[1]) : s_red[0];

    float acc0 = 0.f, acc1 = 0.f, wsum = 0.f;
    for (int j0 = 0; j0 < pv; j0 += kChunk) {
        const int cnt = min(kChunk, pv - j0);
        __syncthreads();
        for (int jj = tid; jj < cnt; jj += blockDim.x)
            s_w[jj] = l[j0 + jj] * __expf(m[j0 + jj] - mx);
        __syncthreads();
        for (int jj = 0; jj < cnt; ++jj) {
            const float w = s_w[jj];
            wsum += w;
            const float* oj = o + (size_t)(j0 + jj) * head_dim;
            if (tid < head_dim) acc0 = fmaf(w, oj[tid], acc0);
            if (tid + (int)blockDim.x < head_dim) acc1 = fmaf(w, oj[tid + blockDim.x], acc1);
        }
    }
    if (tid < head_dim) store_f32_as<OT>(out, row * head_dim + tid, acc0 / wsum);
    if (tid + (int)blockDim.x < head_dim)
        store_f32_as<OT>(out, row * head_dim + tid + blockDim.x, acc1 / wsum);
}

// ---- dispatch ------------------------------------------------------------------

template <int KT, int QT, int D, int GM>
static hipError_t launch_typed(const DecodeArgs& a) {
    DecodeParams p;
    p.q = static_cast<const uint8_t*>(a.q);
    p.k_cache = static_cast<const uint8_t*>(a.k_cache);
    p.v_cache = static_cast<const uint8_t*>(a.v_cache);
    p.block_tables = a.block_tables;
    p.context_lens = a.context_lens;
    p.num_q_heads = a.num_q_heads;
    p.num_kv_heads = a.num_kv_heads;
    p.group = a.group;
    p.num_blocks = a.num_blocks;
    p.max_blocks_per_seq = a.max_blocks_per_seq;
    p.partition_size = a.partition_size;
    p.num_partitions = a.num_partitions;
    p.qk_scale_log2 = a.scale * (KT == PKV_FP8_E4M3 ? a.k_scale : 1.f) * kLog2e;
    p.v_scale = KT == PKV_FP8_E4M3 ? a.v_scale : 1.f;
    p.ws_m = a.ws_m;
    p.ws_l = a.ws_l;
    p.ws_o = a.ws_o;
    p.out = a.out;
    const size_t smem =
        ((size_t)a.partition_size * GM + kWavesPerGroup * GM * D + 2 * GM) * sizeof(float);
    dim3 grid(a.num_partitions, a.num_kv_heads, a.num_seqs);
    hipLaunchKernelGGL((paged_decode_partition_kernel<KT, QT, D, GM>), grid, dim3(kThreads), smem,
                       a.stream, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.num_partitions == 1) return err;
    dim3 rgrid(a.num_q_heads, a.num_seqs);
    hipLaunchKernelGGL((lse_reduce_kernel<QT>), rgrid, dim3(a.head_dim > 64 ? 128 : 64), 0,
                       a.stream, a.ws_m, a.ws_l, a.ws_o, a.context_lens, a.num_q_heads,
                       a.head_dim, a.num_partitions, a.partition_size,
                       a.max_blocks_per_seq * kBlock, a.out);
    return hipGetLastError();
}

template <int KT, int QT, int D>
static hipError_t launch_group(const DecodeArgs& a) {
    if (a.group <= 1) return launch_typed<KT, QT, D, 1>(a);
    if (a.group <= 2) return launch_typed<KT, QT, D, 2>(a);
    if (a.group <= 4) return launch_typed<KT, QT, D, 4>(a);
    if (a.group <= 6) return launch_typed<KT, QT, D, 6>(a);
    return launch_typed<KT, QT, D, 8>(a);
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
