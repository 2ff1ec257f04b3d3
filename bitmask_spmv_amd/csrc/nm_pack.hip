// nm_pack.hip -- producing the packed operands on gfx950: column norms, Wanda N:M
// selection with bitmask + value packing, and the inverse unpack.
//
// Pages (cited by title and section):
//   "SparseDecoding：只用解码激活校准的稀疏推理" (daiwk.github.io), 核心公式: Wanda score
//       |W_ij| * sqrt(sum_t X_jt^2), top N of every M columns, 32 columns per mask word.
//   "SparseDecoding: Decoding-Aware Pruning ..." (ai.info summary), Methodology Step 2:
//       one bit per column, 32 bits per word, values in increasing column order.
//   "SparseDecoding:解码感知的准确高效大模型剪枝框架" (paper.rainbus.top), 前置知识 N:M;
//       核心方法 (核心创新二): the index formats that the bitmask replaces -- a uint8
//       offset or an int32 column index per kept weight.
//
// All four kernels are offline (run once per weight matrix); they are written for
// bit-exact agreement with a scalar definition rather than for peak bandwidth, but
// still read and write HBM with 16-byte accesses where the layout allows.
#include "nm_device.h"
#include "nm_kernels.h"

namespace nmk {
namespace {

constexpr int kPackThreads = 256;

// ---------------------------------------------------------------- column norm
// One thread per input column; the T loads of a step are coalesced across threads.
__global__ __launch_bounds__(kPackThreads) void col_norm_kernel(const uint16_t *__restrict__ X, int64_t T,
                                                                int64_t K, int64_t ldx, float *__restrict__ n) {
    const int64_t j = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
    if (j >= K) return;
    double s = 0.0;
    for (int64_t t = 0; t < T; ++t) {
        const double v = abs_f32bits_to_f64((uint32_t)X[t * ldx + j] << 16);
        s = s + v * v;  // v*v is exact (16-bit significand), so fusing cannot change s
    }
    n[j] = __uint_as_float(f64_to_f32_rne_bits(sqrt_rn_f64(s)));
}

// ---------------------------------------------------------------- select + pack
// One thread per (row, 32-column word).  Scores are exact fp64 products; a column is
// kept when fewer than N columns of its group precede it in (score desc, column asc).
template <int M>
__global__ __launch_bounds__(kPackThreads) void prune_pack_kernel(const uint16_t *__restrict__ W, int64_t ldw,
                                                                  int64_t R, int64_t KW, const float *__restrict__ n,
                                                                  uint32_t *__restrict__ masks,
                                                                  uint16_t *__restrict__ values) {
    constexpr int N = M / 2;
    const int64_t gid = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
    if (gid >= R * KW) return;
    const int64_t row = gid / KW;
    const int64_t w = gid - row * KW;

    const uint16_t *wrow = W + row * ldw + 32 * w;
    const uint4 *w4 = reinterpret_cast<const uint4 *>(wrow);
    const uint4 *n4 = reinterpret_cast<const uint4 *>(n + 32 * w);
    uint32_t wb[16];
    uint32_t nb[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint4 a = w4[q];
        wb[4 * q + 0] = a.x; wb[4 * q + 1] = a.y; wb[4 * q + 2] = a.z; wb[4 * q + 3] = a.w;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        uint4 a = n4[q];
        nb[4 * q + 0] = a.x; nb[4 * q + 1] = a.y; nb[4 * q + 2] = a.z; nb[4 * q + 3] = a.w;
    }
    double s[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const uint32_t bits = (j & 1) ? (wb[j >> 1] & 0xFFFF0000u) : (wb[j >> 1] << 16);
        s[j] = abs_f32bits_to_f64(bits) * abs_f32bits_to_f64(nb[j]);  // exact
    }
    uint32_t mask = 0;
#pragma unroll
    for (int g = 0; g < 32; g += M) {
#pragma unroll
        for (int j = g; j < g + M; ++j) {
            int ahead = 0;
#pragma unroll
            for (int k = g; k < g + M; ++k) {
                if (k == j) continue;
                ahead += (s[k] > s[j]) || (k < j && s[k] == s[j]);
            }
            mask |= (ahead < N ? 1u : 0u) << j;
        }
    }
    masks[gid] = mask;

    // Kept values in increasing column order: walk the set bits lowest first.
    uint32_t out[8];
    uint32_t mm = mask;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        // "& 31" keeps every access inside the word even for out-of-contract
        // (non-finite) inputs that could leave fewer than 16 bits set.
        const int c0 = __builtin_ctz(mm) & 31;
        mm &= mm - 1;
        const int c1 = __builtin_ctz(mm) & 31;
        mm &= mm - 1;
        out[t] = (uint32_t)wrow[c0] | ((uint32_t)wrow[c1] << 16);
    }
    uint4 *v4 = reinterpret_cast<uint4 *>(values + row * (KW * 16) + 16 * w);
    v4[0] = make_uint4(out[0], out[1], out[2], out[3]);
    v4[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

// ---------------------------------------------------------------- unpack
// One thread per (row, word); the 32 outputs are assembled in a private LDS slot.
__global__ __launch_bounds__(kPackThreads) void unpack_kernel(const uint32_t *__restrict__ masks,
                                                              const uint16_t *__restrict__ values, int64_t R,
                                                              int64_t KW, uint16_t *__restrict__ Wout, int64_t ldw) {
    __shared__ uint4 slot[kPackThreads * 4];
    const int64_t gid = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
    if (gid >= R * KW) return;
    const int64_t row = gid / KW;
    const int64_t w = gid - row * KW;
    uint4 *mine = slot + threadIdx.x * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) mine[q] = make_uint4(0, 0, 0, 0);
    uint16_t *mine16 = reinterpret_cast<uint16_t *>(mine);
    const uint4 *v4 = reinterpret_cast<const uint4 *>(values + row * (KW * 16) + 16 * w);
    const uint4 a = v4[0], b = v4[1];
    const uint32_t vv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t mm = masks[gid];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int c0 = __builtin_ctz(mm) & 31;  // stays in this thread's slot for corrupt masks
        mm &= mm - 1;
        const int c1 = __builtin_ctz(mm) & 31;
        mm &= mm - 1;
        mine16[c0] = (uint16_t)(vv[t] & 0xFFFFu);
        mine16[c1] = (uint16_t)(vv[t] >> 16);
    }
    uint4 *dst = reinterpret_cast<uint4 *>(Wout + row * ldw + 32 * w);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = mine[q];
}

// ---------------------------------------------------------------- index metadata
// One thread per (row, word): the word's 16 set bits, lowest first, become 16 uint8
// offsets within the word (one 16-byte store) or 16 int32 column indices within the row
// (four 16-byte stores).
template <int FMT>
__global__ __launch_bounds__(kPackThreads) void meta_from_mask_kernel(const uint32_t *__restrict__ masks, int64_t R,
                                                                      int64_t KW, uint32_t *__restrict__ meta) {
    const int64_t gid = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
    if (gid >= R * KW) return;
    const int64_t w = gid % KW;
    uint32_t mm = masks[gid];
    uint32_t c[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        c[t] = (uint32_t)__builtin_ctz(mm) & 31u;  // a corrupt mask (< 16 bits) yields 31s
        mm &= mm - 1;
    }
    if constexpr (FMT == kMetaU8) {
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = c[4 * q] | (c[4 * q + 1] << 8) | (c[4 * q + 2] << 16) | (c[4 * q + 3] << 24);
        reinterpret_cast<uint4 *>(meta)[gid] = make_uint4(o[0], o[1], o[2], o[3]);
    } else {
        const uint32_t base = (uint32_t)(32 * w);
        uint4 *dst = reinterpret_cast<uint4 *>(meta) + gid * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            dst[q] = make_uint4(base + c[4 * q], base + c[4 * q + 1], base + c[4 * q + 2], base + c[4 * q + 3]);
    }
}

}  // namespace

hipError_t launch_col_norm(const uint16_t *X, int64_t T, int64_t K, int64_t ldx, float *n, hipStream_t st) {
    const unsigned blocks = (unsigned)((K + kPackThreads - 1) / kPackThreads);
    hipLaunchKernelGGL(col_norm_kernel, dim3(blocks), dim3(kPackThreads), 0, st, X, T, K, ldx, n);
    return hipGetLastError();
}

hipError_t launch_prune_pack(const uint16_t *W, int64_t ldw, int64_t R, int64_t K, const float *n, int N, int M,
                             uint32_t *masks, uint16_t *values, hipStream_t st) {
    (void)N;  // N == M/2 is checked by the caller
    const int64_t KW = K / 32;
    const int64_t units = R * KW;
    const unsigned blocks = (unsigned)((units + kPackThreads - 1) / kPackThreads);
    switch (M) {
    case 4:
        hipLaunchKernelGGL(prune_pack_kernel<4>, dim3(blocks), dim3(kPackThreads), 0, st, W, ldw, R, KW, n, masks,
                           values);
        break;
    case 8:
        hipLaunchKernelGGL(prune_pack_kernel<8>, dim3(blocks), dim3(kPackThreads), 0, st, W, ldw, R, KW, n, masks,
                           values);
        break;
    case 16:
        hipLaunchKernelGGL(prune_pack_kernel<16>, dim3(blocks), dim3(kPackThreads), 0, st, W, ldw, R, KW, n, masks,
                           values);
        break;
    case 32:
        hipLaunchKernelGGL(prune_pack_kernel<32>, dim3(blocks), dim3(kPackThreads), 0, st, W, ldw, R, KW, n, masks,
                           values);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_unpack(const uint32_t *masks, const uint16_t *values, int64_t R, int64_t K, uint16_t *W,
                         int64_t ldw, hipStream_t st) {
    const int64_t KW = K / 32;
    const unsigned blocks = (unsigned)((R * KW + kPackThreads - 1) / kPackThreads);
    hipLaunchKernelGGL(unpack_kernel, dim3(blocks), dim3(kPackThreads), 0, st, masks, values, R, KW, W, ldw);
    return hipGetLastError();
}

hipError_t launch_meta_from_mask(const uint32_t *masks, int64_t R, int64_t K, int fmt, void *meta, hipStream_t st) {
    const int64_t KW = K / 32;
    const unsigned blocks = (unsigned)((R * KW + kPackThreads - 1) / kPackThreads);
    if (fmt == kMetaU8)
        hipLaunchKernelGGL(meta_from_mask_kernel<kMetaU8>, dim3(blocks), dim3(kPackThreads), 0, st, masks, R, KW,
                           (uint32_t *)meta);
    else if (fmt == kMetaI32)
        hipLaunchKernelGGL(meta_from_mask_kernel<kMetaI32>, dim3(blocks), dim3(kPackThreads), 0, st, masks, R, KW,
                           (uint32_t *)meta);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace nmk
