// nm_dense.hip -- same-GPU dense bf16 GEMV baseline on gfx950.
//
// The decode step is a memory-bound matrix-vector product that rereads every weight
// per token ("SparseDecoding:解码感知的准确高效大模型剪枝框架", 前置知识 Prefill 与
// Decoding); this kernel is the dense reference point the sparse kernel is compared
// against, built with the same structure so that the comparison isolates the format:
//   * x staged once per workgroup in LDS (contiguous, read back with 16-byte LDS loads);
//   * a wave owns whole rows (or row slices); lane l reads 16-byte chunk l, l+64, ... of
//     the row with non-temporal loads, so each wave iteration streams 1 KiB contiguously;
//   * four v_dot2_f32_bf16 per chunk per token, fp32 accumulate, wave64 reduction,
//     bf16 round-to-nearest-even store; deterministic split rows as in the sparse kernel.
#include <atomic>

#include "nm_device.h"
#include "nm_kernels.h"

namespace nmk {
namespace {

constexpr int kThreads = 512;

// 1024-thread workgroups (16 waves, at most 64 VGPRs so two fit per CU) when the x slice
// leaves room for only two workgroups per CU, for the instantiations that fit that
// register budget: B = 3 and 4, except the gated-MLP kernel with four chunks per lane at
// B = 4.  The same rule as the sparse kernel's, so the baseline gets the same occupancy.
constexpr bool dense_wide_ok(int B, int U, int EPI) {
    return (B == 3 || B == 4) && !(EPI == kEpiSwiGLU && B == 4 && U == 4);
}
constexpr size_t kLdsCap = 80 * 1024;
constexpr size_t kLdsPerCu = 160 * 1024;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

template <int U>
struct DBatch {
    u32x4 w[U];
    int base;  // first chunk of the batch within the row slice (wave-uniform)
};

// One batch of U 16-byte chunks per lane (chunk base + u*64 + lane) through a raw buffer
// descriptor that starts at the batch and ends at the row slice's `chunks` chunks
// (0 = nothing to load; out-of-range lanes read zeros).  The batch position lives in the
// scalar descriptor and the lane offsets are loop-invariant, so issuing a batch writes
// no vector register but the load destinations.
template <int U>
__device__ __forceinline__ void load_dbatch(DBatch<U> &bt, const u32x4 *wrow, int chunks, int base, int lane) {
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(wrow + base, (int64_t)max(chunks - base, 0) * 16);
#pragma unroll
    for (int u = 0; u < U; ++u)
        bt.w[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, (u * kWave + lane) * 16, 0, kLoadNT);
    bt.base = base;
}

template <int B, int U>
__device__ __forceinline__ void dot_dbatch(const DBatch<U> &bt, const u32x4 *xs4, int ncs, float (&acc)[B]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = bt.base + u * kWave + (int)(threadIdx.x & (kWave - 1));
        const int lc = c < ncs ? c : 0;  // padding lanes carry zero weights
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const u32x4 xv = xs4[b * ncs + lc];
            float a = acc[b];
            a = dot2_bf16(bt.w[u].x, xv.x, a);
            a = dot2_bf16(bt.w[u].y, xv.y, a);
            a = dot2_bf16(bt.w[u].z, xv.z, a);
            a = dot2_bf16(bt.w[u].w, xv.w, a);
            acc[b] = a;
        }
    }
}

// Matrix of the set that owns launch row r (0 <= r < R).  The launcher pads row0 past
// the last matrix with the total row count, so p counts the bounds row0[q] <= r; the
// test is the sign of row0[q] - 1 - r, kept in scalar integer arithmetic (a boolean
// compare is materialised through a vector register, and reusing that register makes
// the wave wait for its in-flight loads).
__device__ __forceinline__ int owner(const DenseSet &set, int r) {
    int p = 0;
#pragma unroll
    for (int q = 1; q < kMaxMats; ++q) p += (int)((uint32_t)(set.row0[q] - 1 - r) >> 31);
    return p;
}

// Matrix and row within it of launch row r (see kEpiSwiGLU for the gated-MLP order).
template <int EPI>
__device__ __forceinline__ void locate(const DenseSet &set, int r, int &p, int &local) {
    if constexpr (EPI == kEpiSwiGLU) {
        p = r & 1;
        local = r >> 1;
    } else if constexpr (EPI == kEpiOne) {
        p = 0;
        local = r;
    } else {
        p = owner(set, r);
        local = r - set.row0[p];
    }
}

// Row finished: wave reduction, then lane 0 writes the bf16 row (gated MLP: h once the up
// row of a pair is done, the gate total kept in gsave until then) or, for a split
// launch, the row's fp32 partial.  `split` and the row parity are integers for the same
// reason as in owner().
//
// The stored data (bf16 bits, or the fp32 bits of a partial) is built in `held`, which the
// row loop pins in vector registers until after the next loads have gone out (hold()):
// a store's data register may not be overwritten until the store has gone (this target
// tracks that with the in-order load counter), so a recycled data register would make
// the wave wait for every load issued before the store.
template <int B, int EPI>
__device__ __forceinline__ void finish_drow(float (&acc)[B], float (&gsave)[B], uint32_t (&held)[B], const DenseSet &set,
                                            int row, int split, int s, int R, int lane, float *partial) {
    const int glu = EPI == kEpiSwiGLU ? 1 - split : 0;  // gated MLP without a split
    const int up = row & 1;
    float val[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const float tot = wave_sum(acc[b]);
        acc[b] = 0.f;
        val[b] = tot;
        if constexpr (EPI == kEpiSwiGLU) {
            gsave[b] = up ? gsave[b] : tot;
            val[b] = glu ? silu_mul(gsave[b], tot) : tot;
        }
    }
    if ((glu & (up ^ 1)) | lane) return;  // a gate row waits for its up row; lane 0 writes
    if (split) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
            held[b] = __float_as_uint(val[b]);
            reinterpret_cast<uint32_t *>(partial)[((int64_t)s * B + b) * R + row] = held[b];
        }
        return;
    }
    int p, local;
    locate<EPI>(set, row, p, local);
#pragma unroll
    for (int b = 0; b < B; ++b) {
        held[b] = f32_to_bf16_rne(val[b]);
        set.y[p][(int64_t)b * set.ldy[p] + local] = (uint16_t)held[b];
    }
}

// Pins the last stored data in vector registers up to this point, past the address
// arithmetic of the loads just issued (see finish_drow).
template <int B>
__device__ __forceinline__ void hold(uint32_t (&held)[B]) {
#pragma unroll
    for (int b = 0; b < B; ++b) asm volatile("" : "+v"(held[b]));
}

// Matrix 0's array and row stride come in as kernel arguments (W0, ldw0), as in the
// sparse kernel: a one-matrix launch uses only those, and the gated MLP (one shared row
// stride) picks between them and matrix 1's array at a fixed argument offset.
template <int U, int EPI>
__device__ __forceinline__ void load_row_dbatch(DBatch<U> &bt, const DenseSet &set, const uint16_t *W0, int64_t ldw0,
                                                int r, int c0, int chunks, int base, int lane) {
    int p, local;
    locate<EPI>(set, r, p, local);
    const uint16_t *wp;
    int64_t ldw;
    if constexpr (EPI == kEpiOne) {
        wp = W0;
        ldw = ldw0;
    } else if constexpr (EPI == kEpiSwiGLU) {
        wp = p ? set.W[1] : W0;
        ldw = ldw0;
    } else {
        wp = set.W[p];
        ldw = set.ldw[p];
    }
    const u32x4 *wrow = reinterpret_cast<const u32x4 *>(wp) + (int64_t)local * (ldw / 8) + c0;
    load_dbatch<U>(bt, wrow, chunks, base, lane);
}

// Leading arguments as in the sparse kernel: what the first batch of loads depends on.
template <int B, int U, int EPI, int NT>
__global__ __launch_bounds__(NT, NT == 1024 ? 8 : 1) void dense_kernel(const uint16_t *W0, int64_t ldw0, int R, int KC,
                                                                       int gx, int split,
                                                                       const uint16_t *__restrict__ x, int64_t ldx,
                                                                       int slice, float *__restrict__ partial,
                                                                       const DenseSet set) {
    extern __shared__ u32x4 xs4[];  // [B][ncs]
    const int s = blockIdx.y;
    const int c0 = s * slice;
    const int ncs = min(slice, KC - c0);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    constexpr int kWaves = NT / kWave;

    // Same flat, software-pipelined walk over (row, batch) as the sparse kernel, with the
    // same row order (row pairs for the gated MLP).
    const int unit = blockIdx.x * kWaves + wave;
    const int row_step = gx * kWaves;
    const int first_row = EPI == kEpiSwiGLU ? 2 * unit : unit;
    const int units = EPI == kEpiSwiGLU ? R / 2 : R;
    const int my_rows = (unit < units ? (units - 1 - unit) / row_step + 1 : 0) * (EPI == kEpiSwiGLU ? 2 : 1);
    const int nb = (ncs + kWave * U - 1) / (kWave * U);
    const int total = my_rows * nb;
    auto next_row = [&](int r) {
        if constexpr (EPI == kEpiSwiGLU) return (r & 1) ? r - 1 + 2 * row_step : r + 1;
        return r + row_step;
    };

    DBatch<U> bufA, bufB;
    int rowA = first_row, biA = 0, rowB = first_row, biB = 0;
    // Stage x; the first round of x loads goes out before batch A's weight loads so that
    // waiting for x never waits for the weights queued behind it.
    {
        // (unconditional loads -- a thread past the end re-reads the last chunk -- and
        // the parts of a round beyond x skipped by a uniform test, as in the sparse
        // kernel's staging: loads under a lane condition were issued one at a time)
        constexpr int kStage = 4;
        const int chunks = B * ncs;
        const int rounds = (chunks + NT - 1) / NT;
        for (int i0 = 0; i0 < chunks || i0 == 0; i0 += NT * kStage) {
            const int left = rounds - i0 / NT;
            u32x4 r[kStage];
#pragma unroll
            for (int j = 0; j < kStage; ++j) {
                if (j > 0 && j >= left) break;
                const int i = min(i0 + j * NT + (int)threadIdx.x, chunks - 1);
                const int b = i / ncs;
                r[j] = reinterpret_cast<const u32x4 *>(x + (int64_t)b * ldx)[c0 + (i - b * ncs)];
            }
            if (i0 == 0) load_row_dbatch<U, EPI>(bufA, set, W0, ldw0, min(rowA, R - 1), c0, total > 0 ? ncs : 0, 0, lane);
#pragma unroll
            for (int j = 0; j < kStage; ++j) {
                if (j > 0 && j >= left) break;
                const int i = i0 + j * NT + (int)threadIdx.x;
                if (i < chunks) xs4[i] = r[j];
            }
        }
    }
    __syncthreads();

    float acc[B], gsave[B];
    uint32_t held[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        acc[b] = gsave[b] = 0.f;
        held[b] = 0u;
    }
    // Whole pairs of batches per iteration, the odd last batch after the loop, and the
    // next batch's loads issued before the current walk waits: the same schedule as the
    // sparse kernel, for the same reasons.
    auto step = [&](int &row, int &bi) {
        if (++bi == nb) {
            bi = 0;
            row = next_row(row);
        }
    };
    int t = 0;
    for (; t + 1 < total; t += 2) {
        rowB = rowA;
        biB = biA;
        step(rowB, biB);
        load_row_dbatch<U, EPI>(bufB, set, W0, ldw0, min(rowB, R - 1), c0, ncs, biB * kWave * U, lane);
        hold(held);
        __builtin_amdgcn_sched_barrier(0);
        dot_dbatch<B, U>(bufA, xs4, ncs, acc);
        if (biA == nb - 1) finish_drow<B, EPI>(acc, gsave, held, set, rowA, split, s, R, lane, partial);
        rowA = rowB;
        biA = biB;
        step(rowA, biA);
        load_row_dbatch<U, EPI>(bufA, set, W0, ldw0, min(rowA, R - 1), c0, t + 2 < total ? ncs : 0, biA * kWave * U, lane);
        hold(held);
        __builtin_amdgcn_sched_barrier(0);
        dot_dbatch<B, U>(bufB, xs4, ncs, acc);
        if (biB == nb - 1) finish_drow<B, EPI>(acc, gsave, held, set, rowB, split, s, R, lane, partial);
    }
    if (t < total) {
        dot_dbatch<B, U>(bufA, xs4, ncs, acc);
        if (biA == nb - 1) finish_drow<B, EPI>(acc, gsave, held, set, rowA, split, s, R, lane, partial);
    }
}

template <int B>
__global__ __launch_bounds__(256) void dense_finish_kernel(const float *__restrict__ partial, int S,
                                                           const DenseSet set) {
    const int R = set.row0[set.P];
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= R) return;
    int p = 0;
    for (int q = 1; q < set.P; ++q)
        if (i >= set.row0[q]) p = q;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float t = 0.f;
        for (int s = 0; s < S; ++s) t += partial[((int64_t)s * B + b) * R + i];
        set.y[p][(int64_t)b * set.ldy[p] + (i - set.row0[p])] = f32_to_bf16_rne(t);
    }
}

template <int B>
__global__ __launch_bounds__(256) void dense_finish_swiglu_kernel(const float *__restrict__ partial, int S,
                                                                  const DenseSet set) {
    const int R2 = set.row0[set.P];
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= R2 / 2) return;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float g = 0.f, u = 0.f;
        for (int s = 0; s < S; ++s) {
            g += partial[((int64_t)s * B + b) * R2 + 2 * i];
            u += partial[((int64_t)s * B + b) * R2 + 2 * i + 1];
        }
        set.y[0][(int64_t)b * set.ldy[0] + i] = f32_to_bf16_rne(silu_mul(g, u));
    }
}

template <int B, int U, int EPI, int NT>
hipError_t allow_lds(size_t bytes) {
    static std::atomic<uint64_t> done{0};
    if (bytes <= 64 * 1024) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = 1ull << (dev & 63);
    if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
    e = hipFuncSetAttribute((const void *)dense_kernel<B, U, EPI, NT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kLdsCap);
    if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

template <int B, int U, int EPI, int NT>
hipError_t launch_bun(const MvPlan &p, const DenseSet &set, int64_t K, const uint16_t *x, int64_t ldx, float *ws,
                      hipStream_t st) {
    hipError_t e = allow_lds<B, U, EPI, NT>(p.lds_bytes);
    if (e != hipSuccess) return e;
    DenseSet padded = set;  // row0 past the last matrix = the total (see owner())
    for (int q = set.P + 1; q <= kMaxMats; ++q) padded.row0[q] = set.row0[set.P];
    hipLaunchKernelGGL((dense_kernel<B, U, EPI, NT>), dim3(p.grid_x, p.splits), dim3(NT), p.lds_bytes, st, set.W[0],
                       set.ldw[0], set.row0[set.P], (int)(K / 8), p.grid_x, p.splits > 1 ? 1 : 0, x, ldx, p.slice, ws,
                       padded);
    e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    const int R = set.row0[set.P];
    if constexpr (EPI == kEpiSwiGLU)
        hipLaunchKernelGGL(dense_finish_swiglu_kernel<B>, dim3((unsigned)((R / 2 + 255) / 256)), dim3(256), 0, st,
                           ws, p.splits, set);
    else
        hipLaunchKernelGGL(dense_finish_kernel<B>, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, st, ws,
                           p.splits, set);
    return hipGetLastError();
}

template <int B, int U, int EPI>
hipError_t launch_bu(const MvPlan &p, const DenseSet &set, int64_t K, const uint16_t *x, int64_t ldx, float *ws,
                     hipStream_t st) {
    if constexpr (dense_wide_ok(B, U, EPI))
        if (p.threads == 1024) return launch_bun<B, U, EPI, 1024>(p, set, K, x, ldx, ws, st);
    return launch_bun<B, U, EPI, kThreads>(p, set, K, x, ldx, ws, st);
}

template <int B, int EPI>
hipError_t launch_b(const MvPlan &p, const DenseSet &set, int64_t K, const uint16_t *x, int64_t ldx, float *ws,
                    hipStream_t st) {
    if (p.unroll >= 4) return launch_bu<B, 4, EPI>(p, set, K, x, ldx, ws, st);
    if (p.unroll == 2) return launch_bu<B, 2, EPI>(p, set, K, x, ldx, ws, st);
    return launch_bu<B, 1, EPI>(p, set, K, x, ldx, ws, st);
}

template <int EPI>
hipError_t launch_e(const MvPlan &p, const DenseSet &set, int64_t K, const uint16_t *x, int64_t ldx, int B,
                    float *ws, hipStream_t st) {
    switch (B) {
    case 1: return launch_b<1, EPI>(p, set, K, x, ldx, ws, st);
    case 2: return launch_b<2, EPI>(p, set, K, x, ldx, ws, st);
    case 3: return launch_b<3, EPI>(p, set, K, x, ldx, ws, st);
    case 4: return launch_b<4, EPI>(p, set, K, x, ldx, ws, st);
    case 5: return launch_b<5, EPI>(p, set, K, x, ldx, ws, st);
    case 6: return launch_b<6, EPI>(p, set, K, x, ldx, ws, st);
    case 7: return launch_b<7, EPI>(p, set, K, x, ldx, ws, st);
    case 8: return launch_b<8, EPI>(p, set, K, x, ldx, ws, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

MvPlan plan_dense(int64_t R, int64_t K, int B, const DeviceInfo &dev, int epi) {
    MvPlan p;
    p.threads = kThreads;
    const int64_t KC = K / 8;  // 16-byte chunks per row
    const int64_t bytes_per_chunk = (int64_t)B * 16;
    size_t cap = kLdsCap;
    if (dev.max_lds_per_block > 0 && (size_t)dev.max_lds_per_block < cap) cap = (size_t)dev.max_lds_per_block;
    int64_t max_slice = (int64_t)cap / bytes_per_chunk;
    if (max_slice >= kWave) max_slice -= max_slice % kWave;
    if (max_slice < 1) max_slice = 1;
    // Split rows across workgroups only when the matrix has too few rows to give
    // every CU a couple of waves: the split costs a second launch, which outweighs
    // the extra parallelism on anything but very short, wide matrices.
    const int64_t cu = dev.num_cu > 0 ? dev.num_cu : 256;
    const int64_t want_rows = cu * 2;
    int64_t splits = (KC + max_slice - 1) / max_slice;
    int64_t by_tasks = R >= want_rows ? 1 : (want_rows + R - 1) / R;
    int64_t max_by_len = KC / (4 * kWave) > 0 ? KC / (4 * kWave) : 1;
    if (by_tasks > max_by_len) by_tasks = max_by_len;
    if (splits < by_tasks) splits = by_tasks;
    int64_t slice = (KC + splits - 1) / splits;
    if (slice > kWave) slice = (slice + kWave - 1) / kWave * kWave;
    if (slice > max_slice) slice = max_slice;
    splits = (KC + slice - 1) / slice;
    p.splits = (int)splits;
    p.slice = (int)slice;
    p.lds_bytes = (size_t)slice * bytes_per_chunk;
    int per_cu = (int)(kLdsPerCu / (p.lds_bytes > 0 ? p.lds_bytes : 1));
    if (per_cu > 4) per_cu = 4;
    if (per_cu < 1) per_cu = 1;
    p.unroll = slice >= 4 * kWave ? 4 : (slice > kWave ? 2 : 1);
    if (per_cu <= 2 && (R + kThreads / kWave - 1) / (kThreads / kWave) * splits >= cu &&
        dense_wide_ok(B, p.unroll, epi))
        p.threads = 1024;
    const int64_t waves = p.threads / kWave;
    int64_t gx = (R + waves - 1) / waves;
    int64_t cap_x = (per_cu * cu + splits - 1) / splits;
    if (gx > cap_x) gx = cap_x;
    if (gx < 1) gx = 1;
    p.grid_x = (int)gx;
    p.ws_bytes = splits > 1 ? (size_t)splits * B * R * sizeof(float) : 0;
    return p;
}

hipError_t launch_dense(const MvPlan &p, const DenseSet &set, int64_t K, const uint16_t *x, int64_t ldx, int B,
                        float *ws, hipStream_t st) {
    if (set.P == 1) return launch_e<kEpiOne>(p, set, K, x, ldx, B, ws, st);
    return launch_e<kEpiNone>(p, set, K, x, ldx, B, ws, st);
}

hipError_t launch_dense_swiglu(const MvPlan &p, const DenseSet &set, int64_t K, const uint16_t *x, int64_t ldx, int B,
                               float *ws, hipStream_t st) {
    if (set.P != 2 || set.row0[2] != 2 * set.row0[1]) return hipErrorInvalidValue;
    return launch_e<kEpiSwiGLU>(p, set, K, x, ldx, B, ws, st);
}

}  // namespace nmk
