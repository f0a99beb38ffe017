// stream_read.hip -- a plain streaming read of device memory: the yardstick
// for the read bandwidth this device delivers to a kernel, reported beside
// the published HBM peak when the decode kernel's bandwidth is judged (the
// ttlab page, section 1, judges decode by the fraction of the rated memory
// bandwidth it reaches). It computes nothing the attention path needs.
//
// The buffer is read once as 32 KiB chunks, chunk c by workgroup c mod the
// grid, each of the 256 threads issuing eight 16-byte nontemporal loads per
// chunk (the decode kernel's load width and cache policy). Every word is
// XORed into one value per workgroup, and each workgroup XORs its value
// into *sink, so no load can be dropped. One workgroup per compute unit is the default:
// a sweep on MI355X over 1..4 workgroups per CU, 4..16 loads per thread,
// contiguous or interleaved chunks and cached loads found this the fastest
// (7.09 TB/s over 1.34 GB; two workgroups 6.8, four 6.2-6.3, cached loads
// 6.3), and more waves only lower the bandwidth delivered.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamLoads = 8;                                    // loads in flight per thread
constexpr uint32_t kStreamChunk = kStreamThreads * 16 * kStreamLoads;  // 32 KiB

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint8_t* src,
                                                                     uint64_t bytes,
                                                                     uint32_t* sink) {
    const uint64_t chunks = (bytes + kStreamChunk - 1) / kStreamChunk;
    uint32_t acc = 0;
    for (uint64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
        const uint64_t off = c * kStreamChunk;
        const uint64_t left = bytes - off;
        // loads past the chunk's valid bytes return zero (buffer bounds)
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(src + off, (uint32_t)(left < kStreamChunk ? left : kStreamChunk));
        u32x4_t a[kStreamLoads];
#pragma unroll
        for (int i = 0; i < kStreamLoads; ++i)
            a[i] = __builtin_amdgcn_raw_buffer_load_b128(
                r, (uint32_t)(i * kStreamThreads + threadIdx.x) * 16u, 0, 2 /* nontemporal */);
#pragma unroll
        for (int i = 0; i < kStreamLoads; ++i) acc ^= a[i][0] ^ a[i][1] ^ a[i][2] ^ a[i][3];
    }
#pragma unroll
    for (int sh = 1; sh < kWave; sh <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, sh, kWave);
    // one atomic per workgroup: atomics on one address are serialised, and
    // one per wave cost ~10 ns each on MI355X (1024 of them, the default
    // grid's waves, added up to ~10 us to a 147 MB read)
    __shared__ uint32_t wave_acc[kStreamThreads / kWave];
    if ((threadIdx.x & (kWave - 1)) == 0) wave_acc[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
#pragma unroll
        for (int i = 0; i < kStreamThreads / kWave; ++i) x ^= wave_acc[i];
        atomicXor(sink, x);
    }
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int num_workgroups,
                              hipStream_t stream) {
    if (num_workgroups == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return hipErrorInvalidDevice;
        num_workgroups = cus;
    }
    const uint64_t chunks = (bytes + kStreamChunk - 1) / kStreamChunk;
    if ((uint64_t)num_workgroups > chunks) num_workgroups = (int)chunks;
    if (num_workgroups < 1) num_workgroups = 1;
    hipLaunchKernelGGL(stream_read_kernel, dim3(num_workgroups), dim3(kStreamThreads), 0, stream,
                       static_cast<const uint8_t*>(src), (uint64_t)bytes, sink);
    return hipGetLastError();
}

}  // namespace pkv
