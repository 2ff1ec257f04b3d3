// nm_spmv_unstructured.hip -- matrix-vector product of 50% unstructured rows on gfx950.
//
// What it computes (pages cited by title and section):
//   "SparseDecoding: Decoding-Aware Pruning ..." (ai.info summary), Methodology Steps 2-4:
//     the same encoding as the N:M kernel (one bit per column, kept values in increasing
//     column order) for the pages' other 50% setting, unstructured sparsity, where a row
//     keeps half of its weights but a 32-bit word may hold anywhere from 0 to 32 of them.
//     Step 3 names exactly this case as the one the fixed 16-step walk does not cover:
//     the number of traversal steps now differs between words.
//
// gfx950 design:
//   * x in LDS exactly as in the N:M kernel (shared staging and layout).
//   * one mask word per lane (lane l <-> word l of a 64-word strip, in word order); the
//     wave's popcounts are prefix-summed across lanes (shuffles) to give every lane the
//     offset of its word's values, and their total is the strip's value count n.
//   * a strip's values are one contiguous run of the row's packed values; it is loaded
//     with 16-byte loads that are contiguous across the wave, through a buffer
//     descriptor that ends at the run (loads past it return zeros and move no data), and
//     written to a per-wave LDS window from which lanes read their own values.
//   * each lane walks its word two set bits at a time (lowest set bit, clear it) and
//     feeds v_dot2_f32_bf16 with the value pair; the wave runs as many pair steps as its
//     fullest word needs (lanes whose word ran out contribute zeros).
//   * software pipeline: while strip t is walked, the values of strip t+1 (whose masks
//     arrived one iteration earlier) and the masks of strip t+2 are in flight.
//   * rows are balanced by construction (K/2 kept per row); a wave owns whole rows (or
//     row slices, whose value offset is the popcount of the masks before the slice).
#include "nm_device.h"
#include "nm_kernels.h"
#include "nm_spmv_common.h"

namespace nmk {
namespace {

constexpr int kUThreads = 512;                 // 8 waves per workgroup
constexpr int kWinChunks = 264;                // per-wave window: 16-byte chunks (>= 7 + 2048 + 34 values)
constexpr int kWinBytes = kWinChunks * 16;
constexpr int kValLoads = (kWinChunks + kWave - 1) / kWave;  // 16-byte loads per lane for one strip (5)
constexpr int kLead = 4;                       // zero dwords in front of x (see the walk)
constexpr size_t kULdsCap = 80 * 1024;
constexpr size_t kULdsPerCu = 160 * 1024;

__device__ __forceinline__ uint32_t load_mask(const uint32_t *masks, int row, int KW, int w0, int nws, int base,
                                              int lane) {
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(masks + (int64_t)row * KW + w0, (int64_t)nws * 4);
    return __builtin_amdgcn_raw_buffer_load_b32(rm, (base + lane) * 4, 0, kLoadNT);
}

// Exclusive prefix sum of v over the wave (lane order) and the wave total, with DPP:
// shifts by 1, 2, 4, 8 inside each row of 16 lanes (lanes whose source lies outside the
// row add 0), then lane 15 of rows 0 and 2 added into rows 1 and 3, then lane 31 into
// rows 2 and 3.
__device__ __forceinline__ int wave_excl_scan(int v, int lane, int &total) {
    int incl = v;
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, true);  // row_shr:1
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, true);  // row_shr:2
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, true);  // row_shr:4
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, true);  // row_shr:8
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x142, 0xA, 0xF, false);  // row_bcast:15
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x143, 0xC, 0xF, false);  // row_bcast:31
    (void)lane;
    // the total is wave-uniform: keep it in a scalar register (buffer descriptors built
    // from it stay scalar)
    total = __builtin_amdgcn_readlane(incl, kWave - 1);
    return incl - v;
}

// Issues the loads of a strip's values: [vb, vb + n) of the row's K/2 packed values,
// from the enclosing 16-byte chunk on; chunk c goes to lane c % 64, load c / 64.  Only
// the loads that can carry data are issued (the count is wave-uniform); registers of the
// others are zeroed.
__device__ __forceinline__ void load_values(u32x4 (&v)[kValLoads], const uint16_t *vrow, int half_k, int vb, int n,
                                            int lane) {
    const int a0 = vb & ~7;                                  // first value of the first chunk
    int end = (vb + n - a0) * 2;                             // bytes needed from a0
    end = (end + 15) & ~15;
    const int room = (half_k - a0) * 2;                      // never past the row's values
    if (end > room) end = room > 0 ? room : 0;
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vrow + a0, end);
    const int loads = (end / 16 + kWave - 1) / kWave;
#pragma unroll
    for (int q = 0; q < kValLoads; ++q)
        v[q] = q < loads ? __builtin_amdgcn_raw_buffer_load_b128(rv, (q * kWave + lane) * 16, 0, kLoadNT)
                         : u32x4{0u, 0u, 0u, 0u};
}

// Value count offset of a row slice starting at word w0: popcount of the row's earlier
// masks (only for split rows).
__device__ __forceinline__ int slice_value_base(const uint32_t *masks, int row, int KW, int w0, int lane) {
    int acc = 0;
    for (int b = 0; b < w0; b += kWave) {
        const uint32_t m = load_mask(masks, row, KW, 0, w0, b, lane);
        acc += __builtin_popcount(m);
    }
    int total;
    wave_excl_scan(acc, lane, total);
    return total;
}

template <int B>
__global__ __launch_bounds__(kUThreads) void spmv_unstructured_kernel(const uint32_t *__restrict__ masks,
                                                                      const uint16_t *__restrict__ values, int R,
                                                                      int KW, const uint16_t *__restrict__ x,
                                                                      int64_t ldx, uint16_t *__restrict__ y,
                                                                      int64_t ldy, float *__restrict__ partial,
                                                                      int slice) {
    constexpr int kBlk = XLayout<B>::kBlk;
    constexpr int kWaves = kUThreads / kWave;
    extern __shared__ uint32_t lds[];  // [kLead zeros][nws][kBlk] x, then kWaves windows of kWinBytes
    uint32_t *xs = lds + kLead;
    const int s = blockIdx.y;
    const int w0 = s * slice;
    const int nws = min(slice, KW - w0);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int half_k = KW * 16;
    uint16_t *win = reinterpret_cast<uint16_t *>(reinterpret_cast<uint8_t *>(xs) +
                                                 (((size_t)nws * kBlk * 4 + 15) & ~(size_t)15) +
                                                 (size_t)wave * kWinBytes);

    const int first_row = blockIdx.x * kWaves + wave;
    const int row_step = gridDim.x * kWaves;
    const int nb = (nws + kWave - 1) / kWave;
    const int my_rows = first_row < R ? (R - 1 - first_row) / row_step + 1 : 0;
    const int total = my_rows * nb;

    // Prologue: masks of strip 0 go out with the first round of x loads.
    uint32_t mA = 0, mB = 0;  // masks of the strips in turn (no register copies of loads)
    stage_x<B, kUThreads>(xs, x, ldx, w0, nws, [&] {
        if (total > 0) mA = load_mask(masks, first_row, KW, w0, nws, 0, lane);
    });
    // Zero the dwords in front of x and the pad dwords of every block: a lane whose word
    // has run out of set bits scans -1, which addresses the pad just before its block
    // (or the leading zeros), so it multiplies by an x of exactly 0.
    {
        constexpr int kData = XLayout<B>::S == 1 ? 16 : 16 * XLayout<B>::S;
        constexpr int kPad = kBlk - kData;
        if (threadIdx.x < kLead) lds[threadIdx.x] = 0u;
        for (int w = threadIdx.x; w < nws; w += kUThreads)
#pragma unroll
            for (int q = 0; q < kPad; ++q) xs[w * kBlk + kData + q] = 0u;
    }
    __syncthreads();
    if (total == 0) return;

    // Strip bookkeeping: scalar (row, strip, value base, count) plus this lane's offset.
    int row = first_row, bi = 0, vb = 0, n = 0, off = 0;
    u32x4 vals[kValLoads];
    vb = w0 > 0 ? slice_value_base(masks, row, KW, w0, lane) : 0;
    off = wave_excl_scan(__builtin_popcount(mA), lane, n);
    load_values(vals, values + (int64_t)row * half_k, half_k, vb, n, lane);
    if (total > 1) mB = load_mask(masks, nb > 1 ? row : row + row_step, KW, w0, nws, nb > 1 ? kWave : 0, lane);

    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;

    // One strip: m_this holds its mask (arrived), m_other the next strip's (in flight).
    // The walk works on a copy of m_this, so m_this can take the masks of the strip
    // after next before the walk starts.
    auto step = [&](uint32_t &m_this, uint32_t &m_other, int t) {
        // values of strip t: fill the window
#pragma unroll
        for (int q = 0; q < kValLoads; ++q) {
            const int c = q * kWave + lane;
            if (c < kWinChunks) reinterpret_cast<u32x4 *>(win)[c] = vals[q];
        }
        const uint32_t m_walk = m_this;
        const int vi0 = (vb & 7) + off;  // window element of this lane's first value
        const int word = bi * kWave + lane;
        const uint32_t *blk = xs + (word < nws ? word : 0) * kBlk;
        const int row_cur = row;
        const bool row_ends = bi == nb - 1;

        // next strip: scan its masks, send out its value loads and the strip-after-next masks
        if (t + 1 < total) {
            int nbi = bi + 1, nrow = row, nvb = vb + n;
            if (nbi == nb) {
                nbi = 0;
                nrow += row_step;
                nvb = w0 > 0 ? slice_value_base(masks, nrow, KW, w0, lane) : 0;
            }
            off = wave_excl_scan(__builtin_popcount(m_other), lane, n);
            load_values(vals, values + (int64_t)nrow * half_k, half_k, nvb, n, lane);
            if (t + 2 < total) {
                int r2 = nrow, b2 = nbi + 1;
                if (b2 == nb) {
                    b2 = 0;
                    r2 += row_step;
                }
                m_this = load_mask(masks, r2, KW, w0, nws, b2 * kWave, lane);
            }
            row = nrow;
            bi = nbi;
            vb = nvb;
        }
        // window writes before the reads of other lanes' chunks (one wave; the fence keeps
        // the compiler from reordering the LDS accesses across it)
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

        // walk strip t: two set bits per step, values from the window.  A lane past its
        // word's last bit scans -1 (__builtin_ctzg with fallback -1 is the hardware's
        // lowest-set-bit scan), reads the zero pad in front of its block as x and so adds
        // exactly 0 whatever finite value the window holds at its (then foreign) index; the
        // window is rewritten in full for every strip and sized for the largest index.
        // Four pairs per check of the wave's remaining bits, so the LDS reads of several
        // pairs overlap; a word has at most 16 pairs, a multiple of four, so no lane reads
        // past the index bound the window is sized for.
        uint32_t mm = m_walk;
        int vi = vi0;
        while (__builtin_amdgcn_ballot_w64(mm != 0)) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c0 = __builtin_ctzg(mm, -1);
                mm &= mm - 1;
                const int c1 = __builtin_ctzg(mm, -1);
                mm &= mm - 1;
                // the pair (vi, vi+1) from the two aligned dwords around it (a dword read at
                // a 2-byte offset would be a slow misaligned LDS access)
                const uint32_t *w32 = reinterpret_cast<const uint32_t *>(win) + (vi >> 1);
                const uint32_t pr = __builtin_amdgcn_alignbit(w32[1], w32[0], (uint32_t)(vi & 1) * 16u);
                dot_pair<B>(pr, blk, c0, c1, acc);
                vi += 2;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // reads before the next strip's writes

        if (row_ends) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float tot = wave_sum(acc[b]);
                acc[b] = 0.f;
                if (lane == 0) {
                    if (gridDim.y == 1)
                        y[(int64_t)b * ldy + row_cur] = f32_to_bf16_rne(tot);
                    else
                        partial[((int64_t)s * B + b) * R + row_cur] = tot;
                }
            }
        }
    };
    for (int t = 0; t < total; t += 2) {
        step(mA, mB, t);
        if (t + 1 >= total) break;
        step(mB, mA, t + 1);
    }
}

template <int B>
__global__ __launch_bounds__(256) void unstructured_finish_kernel(const float *__restrict__ partial, int S, int R,
                                                                  uint16_t *__restrict__ y, int64_t ldy) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= R) return;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float t = 0.f;
        for (int s = 0; s < S; ++s) t += partial[((int64_t)s * B + b) * R + i];
        y[(int64_t)b * ldy + i] = f32_to_bf16_rne(t);
    }
}

template <int B>
hipError_t launch_u(const MvPlan &p, const uint32_t *masks, const uint16_t *values, int64_t R, int64_t K,
                    const uint16_t *x, int64_t ldx, uint16_t *y, int64_t ldy, float *ws, hipStream_t st) {
    if (p.lds_bytes > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)spmv_unstructured_kernel<B>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kULdsCap);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(spmv_unstructured_kernel<B>, dim3(p.grid_x, p.splits), dim3(kUThreads), p.lds_bytes, st,
                       masks, values, (int)R, (int)(K / 32), x, ldx, y, ldy, ws, p.slice);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    hipLaunchKernelGGL(unstructured_finish_kernel<B>, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, st, ws,
                       p.splits, (int)R, y, ldy);
    return hipGetLastError();
}

}  // namespace

MvPlan plan_spmv_unstructured(int64_t R, int64_t K, int B, const DeviceInfo &dev) {
    MvPlan p;
    p.threads = kUThreads;
    const int64_t KW = K / 32;
    const int64_t bytes_per_word = (int64_t)spmv_lds_per_word(B);
    const int64_t windows = (int64_t)(kUThreads / kWave) * kWinBytes;
    size_t cap = kULdsCap;
    if (dev.max_lds_per_block > 0 && (size_t)dev.max_lds_per_block < cap) cap = (size_t)dev.max_lds_per_block;
    int64_t max_slice = ((int64_t)cap - windows - 16 - kLead * 4) / bytes_per_word;
    if (max_slice >= kWave) max_slice -= max_slice % kWave;
    if (max_slice < 1) max_slice = 1;
    // Same policy as the N:M planner: split only when LDS forces it or rows are few.
    const int64_t cu = dev.num_cu > 0 ? dev.num_cu : 256;
    int64_t splits = (KW + max_slice - 1) / max_slice;
    int64_t by_tasks = R >= cu * 2 ? 1 : (cu * 2 + R - 1) / R;
    const int64_t max_by_len = KW / kWave > 0 ? KW / kWave : 1;
    if (by_tasks > max_by_len) by_tasks = max_by_len;
    if (splits < by_tasks) splits = by_tasks;
    int64_t slice = (KW + splits - 1) / splits;
    if (slice > kWave) slice = (slice + kWave - 1) / kWave * kWave;
    if (slice > max_slice) slice = max_slice;
    splits = (KW + slice - 1) / slice;
    p.splits = (int)splits;
    p.slice = (int)slice;
    p.lds_bytes = (size_t)kLead * 4 + (((size_t)slice * bytes_per_word + 15) & ~(size_t)15) + (size_t)windows;
    int per_cu = (int)(kULdsPerCu / p.lds_bytes);
    if (per_cu > 8) per_cu = 8;
    if (per_cu < 1) per_cu = 1;
    const int64_t waves = kUThreads / kWave;
    int64_t gx = (R + waves - 1) / waves;
    const int64_t cap_x = (per_cu * cu + splits - 1) / splits;
    if (gx > cap_x) gx = cap_x;
    if (gx < 1) gx = 1;
    p.grid_x = (int)gx;
    p.unroll = 1;
    p.ws_bytes = splits > 1 ? (size_t)splits * B * R * sizeof(float) : 0;
    return p;
}

hipError_t launch_spmv_unstructured(const MvPlan &p, const uint32_t *masks, const uint16_t *values, int64_t R,
                                    int64_t K, const uint16_t *x, int64_t ldx, int B, uint16_t *y, int64_t ldy,
                                    float *ws, hipStream_t st) {
    switch (B) {
    case 1: return launch_u<1>(p, masks, values, R, K, x, ldx, y, ldy, ws, st);
    case 2: return launch_u<2>(p, masks, values, R, K, x, ldx, y, ldy, ws, st);
    case 3: return launch_u<3>(p, masks, values, R, K, x, ldx, y, ldy, ws, st);
    case 4: return launch_u<4>(p, masks, values, R, K, x, ldx, y, ldy, ws, st);
    case 5: return launch_u<5>(p, masks, values, R, K, x, ldx, y, ldy, ws, st);
    case 6: return launch_u<6>(p, masks, values, R, K, x, ldx, y, ldy, ws, st);
    case 7: return launch_u<7>(p, masks, values, R, K, x, ldx, y, ldy, ws, st);
    case 8: return launch_u<8>(p, masks, values, R, K, x, ldx, y, ldy, ws, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace nmk
