// nm_stream.hip -- measurement aid: a plain streaming read of one buffer.
//
// The matrix-vector kernels are judged against the memory system's bandwidth; this
// kernel shows what a launch that only reads delivers under the same conditions (the
// same 16-byte non-temporal buffer loads, the same grid of 512-thread workgroups, the
// same rotation over distinct buffers).  Every dword read is XOR-folded and one fold per
// wave is written, so the loads cannot be dropped and the result is checkable: the XOR of
// all folds equals the XOR of all dwords of the buffer.
#include "nm_device.h"
#include "nm_kernels.h"

namespace nmk {
namespace {

constexpr int kSThreads = 512;
constexpr int kSWaves = kSThreads / kWave;
constexpr int kSUnroll = 2;         // 1 KiB wave loads per unit; two units in flight per wave
constexpr int kSMaxGroups = 1024;   // four 512-thread workgroups per CU on 256 CUs
constexpr uint32_t kSUnitBytes = 2048; // one unit = two 1 KiB wave loads

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

// The buffer is cut into 2 KiB units (one 16-byte load per lane for each KiB); wave gw of
// W takes units gw, gw + W, gw + 2W, ..., so the waves of a workgroup sweep adjacent
// units, as the matrix-vector kernels' waves sweep adjacent rows.  The grid gives every
// wave at least two units, up to four 512-thread workgroups per CU.  Two units are in
// flight per wave: the next unit of a buffer is issued right after that buffer is
// folded.  The loop has a single exit at its top (the second buffer past the end reads
// zeros, which leave the fold as it is), and the wave index is made wave-uniform, so
// the loop runs on scalar registers and every wait covers one unit only.  The grid size
// is an argument (preloaded with the others) rather than a dispatch-packet read, and each
// wave writes its own fold (no workgroup barrier at the end).
__global__ __launch_bounds__(kSThreads) void stream_read_kernel(const uint8_t *__restrict__ buf, uint32_t bytes,
                                                                uint32_t *__restrict__ sink, uint32_t grid) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t gw = blockIdx.x * kSWaves + wave;
    const uint32_t W = grid * kSWaves;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(buf, bytes);  // past the end: zeros
    constexpr uint32_t U = kSUnroll * 1024u;                   // one unit
    const uint32_t units = (bytes + U - 1) / U;                // offsets stay below 2^31 + 2^25
    uint32_t ua = gw, ub = gw + W;
    u32x4 a[kSUnroll], b[kSUnroll];
    load_group(a, rs, ua * U + lane * 16u);
    load_group(b, rs, ub * U + lane * 16u);
    uint32_t fold = 0;
    while (ua < units) {
        fold ^= fold_group(a);
        ua = ub + W;
        load_group(a, rs, ua * U + lane * 16u);
        __builtin_amdgcn_sched_barrier(0);
        fold ^= fold_group(b);
        ub = ua + W;
        load_group(b, rs, ub * U + lane * 16u);
        __builtin_amdgcn_sched_barrier(0);
    }
    // XOR over the wave: within rows of 16 lanes by DPP, then the four row results (a
    // cross-lane shuffle through LDS here cost 0.2 us at the end of every launch)
    fold ^= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)fold, 0xB1, 0xF, 0xF, false);   // quad_perm(1,0,3,2)
    fold ^= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)fold, 0x4E, 0xF, 0xF, false);   // quad_perm(2,3,0,1)
    fold ^= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)fold, 0x141, 0xF, 0xF, false);  // row_half_mirror
    fold ^= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)fold, 0x140, 0xF, 0xF, false);  // row_mirror
    const uint32_t wf = (uint32_t)__builtin_amdgcn_readlane((int)fold, 0) ^ (uint32_t)__builtin_amdgcn_readlane((int)fold, 16) ^
                        (uint32_t)__builtin_amdgcn_readlane((int)fold, 32) ^ (uint32_t)__builtin_amdgcn_readlane((int)fold, 48);
    if (lane == 0) sink[gw] = wf;
}

}  // namespace

size_t stream_read_groups(size_t bytes) {
    // two units per wave at least: a launch over a small buffer runs fewer, fuller waves
    // (19 MB: 5.60 -> 4.98 us; 66 MB and up within 1%)
    const size_t per_group = (size_t)kSWaves * kSUnitBytes * 2;
    size_t g = (bytes + per_group - 1) / per_group;
    if (g > (size_t)kSMaxGroups) g = kSMaxGroups;
    return g < 1 ? 1 : g;
}

size_t stream_read_waves(size_t bytes) { return stream_read_groups(bytes) * kSWaves; }

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st) {
    const unsigned grid = (unsigned)stream_read_groups(bytes);
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kSThreads), 0, st, static_cast<const uint8_t *>(buf),
                       (uint32_t)bytes, sink, grid);
    return hipGetLastError();
}

}  // namespace nmk
