// nm_stream.hip -- measurement aid: a plain streaming read of one buffer.
//
// The matrix-vector kernels are judged against the memory system's bandwidth; this
// kernel shows what a launch that only reads delivers under the same conditions (the
// same 16-byte non-temporal buffer loads of 512-thread workgroups, the same rotation over
// distinct buffers), in the grid shape that reads fastest.  Every dword read is XOR-folded and one fold per
// wave is written, so the loads cannot be dropped and the result is checkable: the XOR of
// all folds equals the XOR of all dwords of the buffer.
#include "nm_device.h"
#include "nm_kernels.h"

namespace nmk {
namespace {

constexpr int kSThreads = 512;
constexpr int kSWaves = kSThreads / kWave;
constexpr uint32_t kSUnitBytes = 1024;  // one unit = one 16-byte load per lane, 1 KiB per wave
constexpr int kSMaxGroups = 256;        // one 8-wave workgroup per CU on 256 CUs

// The buffer is cut into 1 KiB units; wave gw of W takes units gw, gw + W, gw + 2W, ...,
// so the waves of a workgroup read adjacent units.  D units are in flight per wave: the
// next unit of a register set is issued right after that set is folded.  One 8-wave
// workgroup per CU with 3 or 4 units in flight per wave (24-32 KiB per CU) reads faster
// than more, fuller workgroups: a sweep of 256-1024-thread workgroups, 1-4 KiB units, 2-4
// units in flight and 1-8 workgroups per CU put this shape first at 19, 66, 132 and
// 264 MB (66 MB: 75.5% of 8 TB/s against 73.9% with four 8-wave workgroups per CU and
// two 2 KiB units in flight per wave; 264 MB: 86.5% against 82.5%).  The loop has a single
// exit at its top (loads past the end read zeros, which leave the fold as it is), and the
// wave index is wave-uniform, so the loop runs on scalar registers and every wait covers
// one unit only.  The grid size is an argument (preloaded with the others), and each wave
// writes its own fold (no workgroup barrier at the end).
template <int D>
__global__ __launch_bounds__(kSThreads) void stream_read_kernel(const uint8_t *__restrict__ buf, uint32_t bytes,
                                                                uint32_t *__restrict__ sink, uint32_t grid) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t gw = blockIdx.x * kSWaves + wave;
    const uint32_t W = grid * kSWaves;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(buf, bytes);       // past the end: zeros
    const uint32_t units = (bytes + kSUnitBytes - 1) / kSUnitBytes;  // offsets stay below 2^31 + 2^24
    u32x4 v[D];
    uint32_t u[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        u[d] = gw + d * W;
        v[d] = __builtin_amdgcn_raw_buffer_load_b128(rs, u[d] * kSUnitBytes + lane * 16u, 0, kLoadNT);
    }
    uint32_t fold = 0;
    while (u[0] < units) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            fold ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
            u[d] = u[d == 0 ? D - 1 : d - 1] + W;
            v[d] = __builtin_amdgcn_raw_buffer_load_b128(rs, u[d] * kSUnitBytes + lane * 16u, 0, kLoadNT);
            __builtin_amdgcn_sched_barrier(0);
        }
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
    // at least two units per wave: a launch over a small buffer runs fewer, fuller waves
    const size_t units = (bytes + kSUnitBytes - 1) / kSUnitBytes;
    size_t g = units / (2 * kSWaves);
    if (g > (size_t)kSMaxGroups) g = kSMaxGroups;
    return g < 1 ? 1 : g;
}

size_t stream_read_waves(size_t bytes) { return stream_read_groups(bytes) * kSWaves; }

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st) {
    const unsigned grid = (unsigned)stream_read_groups(bytes);
    // four units in flight per wave for 40-200 MB (the MLP layers' sizes), three otherwise
    // (19 MB: 4.80 vs 4.95 us; 66 MB: 10.94 vs 11.17 us; 264 MB: 38.2 vs 38.5 us)
    if (bytes >= (size_t)40e6 && bytes <= (size_t)200e6)
        hipLaunchKernelGGL(stream_read_kernel<4>, dim3(grid), dim3(kSThreads), 0, st, static_cast<const uint8_t *>(buf),
                           (uint32_t)bytes, sink, grid);
    else
        hipLaunchKernelGGL(stream_read_kernel<3>, dim3(grid), dim3(kSThreads), 0, st, static_cast<const uint8_t *>(buf),
                           (uint32_t)bytes, sink, grid);
    return hipGetLastError();
}

}  // namespace nmk
