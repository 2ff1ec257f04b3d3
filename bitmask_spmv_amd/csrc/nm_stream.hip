// nm_stream.hip -- measurement aid: a plain streaming read of one buffer.
//
// The matrix-vector kernels are judged against the memory system's bandwidth; this
// kernel shows what a launch that only reads delivers under the same conditions (the
// same 16-byte non-temporal buffer loads, the same grid of 512-thread workgroups, the
// same rotation over distinct buffers).  Every dword read is XOR-folded and one fold per
// workgroup is written, so the loads cannot be dropped and the result is checkable: the
// XOR of all folds equals the XOR of all dwords of the buffer.
#include "nm_device.h"
#include "nm_kernels.h"

namespace nmk {
namespace {

constexpr int kSThreads = 512;
constexpr int kSWaves = kSThreads / kWave;
constexpr int kSUnroll = 2;         // 1 KiB wave loads per group; two groups in flight per wave
constexpr int kSMaxGroups = 1024;   // four 512-thread workgroups per CU on 256 CUs
constexpr uint32_t kSUnitBytes = 4096; // one unit = two groups of two 1 KiB wave loads

template <int U>
__device__ __forceinline__ void load_group(u32x4 (&v)[U], __amdgpu_buffer_rsrc_t rs, uint32_t off) {
#pragma unroll
    for (int u = 0; u < U; ++u)  // past the buffer: zeros, which leave the fold as it is
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + u * 1024u, 0, kLoadNT);
}

template <int U>
__device__ __forceinline__ uint32_t fold_group(const u32x4 (&v)[U]) {
    uint32_t f = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) f ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    return f;
}

// The buffer is cut into 4 KiB units; wave gw of W takes units gw, gw + W, gw + 2W, ...,
// so the waves of a workgroup sweep adjacent units, as the matrix-vector kernels' waves
// sweep adjacent rows (measured faster than one contiguous segment per wave: 20.8 vs
// 22.4 us for 132 MB).  Each unit is two groups of kSUnroll 1 KiB wave loads (16 bytes
// per lane); the next unit's group is issued before the current one is consumed.
__global__ __launch_bounds__(kSThreads) void stream_read_kernel(const uint8_t *__restrict__ buf, uint32_t bytes,
                                                                uint32_t *__restrict__ sink) {
    __shared__ uint32_t part[kSWaves];
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t gw = blockIdx.x * kSWaves + threadIdx.x / kWave;
    const uint32_t W = gridDim.x * kSWaves;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(buf, bytes);  // past the end: zeros
    constexpr uint32_t G = kSUnroll * 1024u;                   // one group = half a unit
    const uint32_t ustride = W * 2 * G;  // <= 32 MiB; offsets stay below 2^31 + 2^26
    uint32_t u0 = gw * 2 * G;
    u32x4 a[kSUnroll], b[kSUnroll];
    load_group(a, rs, u0 + lane * 16u);
    load_group(b, rs, u0 + G + lane * 16u);
    uint32_t fold = 0;
    for (uint32_t off = u0; off < bytes; off += ustride) {
        fold ^= fold_group(a);
        load_group(a, rs, off + ustride + lane * 16u);
        __builtin_amdgcn_sched_barrier(0);
        fold ^= fold_group(b);
        load_group(b, rs, off + ustride + G + lane * 16u);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) fold ^= (uint32_t)__shfl_xor((int)fold, d, kWave);
    if (lane == 0) part[threadIdx.x / kWave] = fold;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t f = 0;
#pragma unroll
        for (int w = 0; w < kSWaves; ++w) f ^= part[w];
        sink[blockIdx.x] = f;
    }
}

}  // namespace

size_t stream_read_groups(size_t bytes) {
    const size_t per_group = (size_t)kSWaves * kSUnitBytes;  // a unit per wave at least
    size_t g = (bytes + per_group - 1) / per_group;
    if (g > (size_t)kSMaxGroups) g = kSMaxGroups;
    return g < 1 ? 1 : g;
}

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st) {
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)stream_read_groups(bytes)), dim3(kSThreads), 0, st,
                       static_cast<const uint8_t *>(buf), (uint32_t)bytes, sink);
    return hipGetLastError();
}

}  // namespace nmk
