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
//   "SparseDecoding: Decoding-Aware Pruning ..." (ai.info summary), Methodology Step 4:
//       50% unstructured sparsity -- each row keeps its K/2 highest scores, same encoding.
//
// All of these kernels are offline (run once per weight matrix); they are written for
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
        // low_bit keeps every access inside the word even for out-of-contract
        // (non-finite) inputs that could leave fewer than 16 bits set.
        const int c0 = low_bit(mm);
        mm &= mm - 1;
        const int c1 = low_bit(mm);
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
        const int c0 = low_bit(mm);  // stays in this thread's slot for corrupt masks
        mm &= mm - 1;
        const int c1 = low_bit(mm);
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
        c[t] = (uint32_t)low_bit(mm);  // a corrupt mask (< 16 bits) yields 31s
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

// ---------------------------------------------------------------- 50% unstructured rows
// One workgroup per row.  A score |W_ij| * n_j is an exact fp64 product of non-negative
// factors, so the bit patterns of the scores order like the scores: an 8-pass radix
// select (8 bits per pass, most significant first) over the 64-bit patterns finds the
// row's K/2-th largest score T and how many scores equal to T are kept (the lowest
// columns first); block-wide scans then place the mask bits and the kept values.
constexpr int kRowThreads = 256;

__device__ __forceinline__ uint64_t score_key(uint16_t w, uint32_t nbits) {
    const double sc = abs_f32bits_to_f64((uint32_t)w << 16) * abs_f32bits_to_f64(nbits);  // exact
    return (uint64_t)__double_as_longlong(sc);
}

// Exclusive prefix sum over the workgroup (kRowThreads threads); *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *sh, uint32_t *total) {
    const int tid = threadIdx.x;
    sh[tid] = v;
    __syncthreads();
#pragma unroll
    for (int off = 1; off < kRowThreads; off <<= 1) {
        const uint32_t t = tid >= off ? sh[tid - off] : 0u;
        __syncthreads();
        sh[tid] += t;
        __syncthreads();
    }
    const uint32_t incl = sh[tid];
    *total = sh[kRowThreads - 1];
    __syncthreads();
    return incl - v;
}

// The 32 score keys of word w of a row (16-byte loads of W and n).
__device__ __forceinline__ void word_keys(const uint16_t *wrow, const float *n, int64_t w, uint64_t (&key)[32]) {
    const uint4 *w4 = reinterpret_cast<const uint4 *>(wrow + 32 * w);
    const uint4 *n4 = reinterpret_cast<const uint4 *>(n + 32 * w);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 a = w4[q];
        const uint32_t wb[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint4 nb = n4[2 * q + h];
            const uint32_t nn[4] = {nb.x, nb.y, nb.z, nb.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 8 * q + 4 * h + e;  // column within the word
                const uint32_t pair = wb[(4 * h + e) >> 1];
                key[j] = score_key((uint16_t)((j & 1) ? (pair >> 16) : (pair & 0xFFFFu)), nn[e]);
            }
        }
    }
}

__global__ __launch_bounds__(kRowThreads) void prune_pack_unstructured_kernel(const uint16_t *__restrict__ W,
                                                                              int64_t ldw, int64_t KW,
                                                                              const float *__restrict__ n,
                                                                              uint32_t *__restrict__ masks,
                                                                              uint16_t *__restrict__ values) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh[kRowThreads];
    __shared__ uint32_t sel[2];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int64_t K = 32 * KW;
    const uint16_t *wrow = W + row * ldw;
    const uint32_t *nbits = reinterpret_cast<const uint32_t *>(n);

    // 1. radix select of the K/2-th largest key (k = its rank among the keys that share
    //    the bits fixed so far, counted from the largest)
    uint64_t prefix = 0, pmask = 0;
    uint32_t k = (uint32_t)(K / 2);
    for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        hist[tid] = 0u;
        __syncthreads();
        for (int64_t j = tid; j < K; j += kRowThreads) {
            const uint64_t key = score_key(wrow[j], nbits[j]);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid == 0) {
            uint32_t above = 0;
            int d = 255;
            for (; d > 0; --d) {
                if (above + hist[d] >= k) break;
                above += hist[d];
            }
            sel[0] = (uint32_t)d;
            sel[1] = k - above;
        }
        __syncthreads();
        prefix |= (uint64_t)sel[0] << shift;
        pmask |= (uint64_t)0xFFu << shift;
        k = sel[1];
        __syncthreads();
    }
    const uint64_t T = prefix;  // keep every key > T and the first `need` keys == T
    const uint32_t need = k;

    // 2. this thread's contiguous range of words
    const int64_t wpt = (KW + kRowThreads - 1) / kRowThreads;
    const int64_t wb = tid * wpt;
    const int64_t we = wb + wpt < KW ? wb + wpt : KW;
    uint32_t eq = 0;
    for (int64_t w = wb; w < we; ++w) {
        uint64_t key[32];
        word_keys(wrow, n, w, key);
#pragma unroll
        for (int j = 0; j < 32; ++j) eq += key[j] == T ? 1u : 0u;
    }
    uint32_t total;
    uint32_t eq_rank = block_excl_scan(eq, sh, &total);
    uint32_t kept = 0;
    for (int64_t w = wb; w < we; ++w) {
        uint64_t key[32];
        word_keys(wrow, n, w, key);
        uint32_t bits = 0;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            if (key[j] > T) {
                bits |= 1u << j;
            } else if (key[j] == T) {
                if (eq_rank < need) bits |= 1u << j;
                ++eq_rank;
            }
        }
        masks[row * KW + w] = bits;
        kept += (uint32_t)__builtin_popcount(bits);
    }
    // 3. kept values in increasing column order
    uint32_t o = block_excl_scan(kept, sh, &total);
    uint16_t *vrow = values + row * (K / 2);
    for (int64_t w = wb; w < we; ++w) {
        uint32_t mm = masks[row * KW + w];
        while (mm) {
            const int c = __builtin_ctz(mm);
            mm &= mm - 1;
            if (o < (uint32_t)(K / 2)) vrow[o] = wrow[32 * w + c];
            ++o;
        }
    }
}

// Inverse for unstructured rows: one workgroup per row, value offsets by a block scan of
// the words' popcounts.
__global__ __launch_bounds__(kRowThreads) void unpack_unstructured_kernel(const uint32_t *__restrict__ masks,
                                                                          const uint16_t *__restrict__ values,
                                                                          int64_t KW, uint16_t *__restrict__ Wout,
                                                                          int64_t ldw) {
    __shared__ uint32_t sh[kRowThreads];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int64_t K = 32 * KW;
    const int64_t wpt = (KW + kRowThreads - 1) / kRowThreads;
    const int64_t wb = tid * wpt;
    const int64_t we = wb + wpt < KW ? wb + wpt : KW;
    uint32_t cnt = 0;
    for (int64_t w = wb; w < we; ++w) cnt += (uint32_t)__builtin_popcount(masks[row * KW + w]);
    uint32_t total;
    uint32_t o = block_excl_scan(cnt, sh, &total);
    const uint16_t *vrow = values + row * (K / 2);
    for (int64_t w = wb; w < we; ++w) {
        const uint32_t mm = masks[row * KW + w];
        uint32_t out[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            uint32_t lo = 0, hi = 0;
            if (mm & (1u << (2 * q))) lo = o < (uint32_t)(K / 2) ? vrow[o++] : (o++, 0u);
            if (mm & (1u << (2 * q + 1))) hi = o < (uint32_t)(K / 2) ? vrow[o++] : (o++, 0u);
            out[q] = lo | (hi << 16);
        }
        uint4 *dst = reinterpret_cast<uint4 *>(Wout + row * ldw + 32 * w);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = make_uint4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
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

hipError_t launch_prune_pack_unstructured(const uint16_t *W, int64_t ldw, int64_t R, int64_t K, const float *n,
                                         uint32_t *masks, uint16_t *values, hipStream_t st) {
    hipLaunchKernelGGL(prune_pack_unstructured_kernel, dim3((unsigned)R), dim3(kRowThreads), 0, st, W, ldw, K / 32, n,
                       masks, values);
    return hipGetLastError();
}

hipError_t launch_unpack_unstructured(const uint32_t *masks, const uint16_t *values, int64_t R, int64_t K,
                                      uint16_t *W, int64_t ldw, hipStream_t st) {
    hipLaunchKernelGGL(unpack_unstructured_kernel, dim3((unsigned)R), dim3(kRowThreads), 0, st, masks, values, K / 32,
                       W, ldw);
    return hipGetLastError();
}

}  // namespace nmk
