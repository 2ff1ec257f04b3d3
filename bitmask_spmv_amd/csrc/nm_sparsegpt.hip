// nm_sparsegpt.hip -- the OBS / SparseGPT N:M solver on gfx950: layer Hessian,
// damped inverse factor, and column-sequential selection with compensation.
//
// What it computes (pages cited by title and section):
//   "SparseDecoding:解码感知的准确高效大模型剪枝框架" (paper.rainbus.top), 前置知识
//     (训练后剪枝与OBS框架) and 方法步骤详情 第二步: H = 2 X X^T from the calibration
//     activations; a weight's saliency is w_q^2 / (2 [H^-1]_qq); the weight with the
//     smallest saliency is removed and the others are compensated by
//     delta_w = -(w_q / [H^-1]_qq) H^-1_{:,q}, iterated until the target pattern.
//   SparseGPT's published column-sequential schedule (the solver the pages hand their
//     Hessian to): columns are fixed left to right; the inverse Hessian that applies to
//     column i is that of the columns not yet fixed, and all of them are read off the
//     upper Cholesky factor U of H^-1 (H^-1 = U^T U): U[i,i]^2 = [(H_{i:,i:})^-1]_ii and
//     fixing column i moves the later columns by -err_i * U[i, i+1:],
//     err_i = (w_i - w_i_fixed) / U[i,i].  N:M: at the first column of each group of M,
//     every row keeps the N columns of largest w^2 / U[c,c]^2 (ties to the lower column).
//     Damping: H + lambda I, lambda = damp * mean(diag H).
//
// gfx950 design:
//   * H = 2 X^T X is the path's one dense contraction: v_mfma_f64_16x16x4_f64 on bf16
//     activations widened to fp64 in LDS (products of bf16 values are exact in fp64, so
//     H differs from an fp64 reference only by summation order).
//   * U without forming H^-1: with J the index reversal, chol(J H J) = C (lower) gives
//     H = (J C J)(J C J)^T with J C J upper, so U = (J C J)^-1 = J C^-1 J.  Blocked
//     right-looking Cholesky (32-column panels: one-workgroup diagonal factor, panel
//     triangular solve, tiled fp64 trailing update) and blocked lower-triangular inverse.
//   * the column loop works in 32-column blocks (one mask word): one thread per row
//     keeps the block's 32 weights in registers, selects, compensates inside the block
//     against U's 32x32 diagonal block in LDS, writes the mask word, the 16 kept values
//     (rounded once to bf16) and the 32 errors.  SparseGPT's lazy batch update, in
//     batches of 128 columns on the fp64 matrix cores: a block's errors compensate the
//     rest of its batch, and a batch's 128 errors per row compensate every later column
//     in one rank-128 update (one pass over those columns per 128 instead of per 32).
#include "nm_device.h"
#include "nm_kernels.h"

namespace nmk {
namespace {

typedef double v4f64 __attribute__((ext_vector_type(4)));
typedef double v2f64 __attribute__((ext_vector_type(2)));
constexpr int kNB = 32;   // panel / column-block width
constexpr int kLB = 128;  // lazy batch: columns whose compensation of the later columns is applied at once

__device__ __forceinline__ double bf16_to_f64(uint16_t b) { return (double)__uint_as_float((uint32_t)b << 16); }

// fp64 -> bf16, rounded once to nearest even (integer arithmetic on the fp64 pattern).
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
    const int e = (int)(a >> 52) - 1023;  // unbiased exponent (finite inputs)
    if (a == 0) return sign;
    if (e >= -126) {
        // keep 7 fraction bits; the bf16 exponent field is e + 127
        const uint64_t q = a >> 45;                      // [exp11][frac7]
        const uint64_t rem = a & ((1ull << 45) - 1);
        const uint64_t half = 1ull << 44;
        uint64_t r = q + ((rem > half || (rem == half && (q & 1))) ? 1 : 0);
        const int64_t be = (int64_t)(r >> 7) - 1023 + 127;
        if (be >= 255) return (uint16_t)(sign | 0x7F80u);
        return (uint16_t)(sign | (uint16_t)(be << 7) | (uint16_t)(r & 0x7Fu));
    }
    // below 2^-126: multiples of 2^-133; significand with the implicit bit, shifted
    const int sh = 52 - (e + 133);  // bits to drop (>= 46)
    if (sh > 53) return sign;       // below half of 2^-133
    const uint64_t m = (a & ((1ull << 52) - 1)) | (1ull << 52);
    const uint64_t q = m >> sh;
    const uint64_t rem = m & ((1ull << sh) - 1);
    const uint64_t half = 1ull << (sh - 1);
    const uint64_t r = q + ((rem > half || (rem == half && (q & 1))) ? 1 : 0);
    return (uint16_t)(sign | (uint16_t)r);
}

// ---------------------------------------------------------------- Hessian
// H = 2 X^T X.  64x64 tile of H per workgroup (4 waves, 32x32 each = 2x2 MFMA tiles);
// H is symmetric, so only the tiles on and above the diagonal are computed (workgroup
// blockIdx.x walks them row by row) and each is written to both halves.  16 tokens per
// LDS stage, two stage buffers: the next stage's elements of X are loaded into registers
// before the current stage's MFMAs, and one barrier per stage separates the writes of a
// buffer from the reads of the stage before.
constexpr int kHT = 64;
constexpr int kHS = 16;

__global__ __launch_bounds__(256) void hessian_kernel(const uint16_t *__restrict__ X, int64_t T, int64_t K,
                                                      int64_t ldx, double *__restrict__ H, int64_t ldh, int g) {
    __shared__ double As[2][kHS][kHT];
    __shared__ double Bs[2][kHS][kHT];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int bi = 0, rem = (int)blockIdx.x;
    while (rem >= g - bi) {  // row bi of the upper triangle holds g - bi tiles
        rem -= g - bi;
        ++bi;
    }
    const int bj = bi + rem;
    const int64_t i0 = (int64_t)bi * kHT, j0 = (int64_t)bj * kHT;
    const int wi = (wave >> 1) * 32, wj = (wave & 1) * 32;
    v4f64 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = v4f64{0.0, 0.0, 0.0, 0.0};
    const int lt = tid >> 4;         // token within the stage
    const int lc = (tid & 15) * 4;   // first of 4 columns
    double ra[4], rb[4];
    auto fetch = [&](int64_t t0) {
        const int64_t t = t0 + lt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t ci = i0 + lc + e, cj = j0 + lc + e;
            ra[e] = (t < T && ci < K) ? bf16_to_f64(X[t * ldx + ci]) : 0.0;
            rb[e] = (t < T && cj < K) ? bf16_to_f64(X[t * ldx + cj]) : 0.0;
        }
    };
    fetch(0);
    int buf = 0;
    for (int64_t t0 = 0; t0 < T; t0 += kHS) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            As[buf][lt][lc + e] = ra[e];
            Bs[buf][lt][lc + e] = rb[e];
        }
        __syncthreads();
        if (t0 + kHS < T) fetch(t0 + kHS);
#pragma unroll
        for (int s = 0; s < kHS / 4; ++s) {
            const int tk = 4 * s + (lane >> 4);
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const double av = As[buf][tk][wi + 16 * a + (lane & 15)];
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const double bv = Bs[buf][tk][wj + 16 * b + (lane & 15)];
                    acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[a][b], 0, 0, 0);
                }
            }
        }
        buf ^= 1;
    }
    // D layout of the 16x16 f64 tile: lane l, element r -> row l/16 + 4*r, column l%16
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t i = i0 + wi + 16 * a + (lane >> 4) + 4 * r;
                const int64_t j = j0 + wj + 16 * b + (lane & 15);
                if (i < K && j < K) {
                    const double v = 2.0 * acc[a][b][r];
                    H[i * ldh + j] = v;
                    if (bi != bj) H[j * ldh + i] = v;
                }
            }
}

// ---------------------------------------------------------------- damping + reversal
// lambda = damp * mean(diag H) (fixed-order reduction in one workgroup).
__global__ __launch_bounds__(256) void damp_kernel(const double *__restrict__ H, int64_t ldh, int64_t K, double damp,
                                                   double *__restrict__ lam) {
    __shared__ double sh[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < K; i += 256) s += H[i * ldh + i];
    sh[threadIdx.x] = s;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if ((int)threadIdx.x < off) sh[threadIdx.x] += sh[threadIdx.x + off];
        __syncthreads();
    }
    if (threadIdx.x == 0) *lam = damp * (sh[0] / (double)K);
}

// A = J (H + lambda I) J, row-major [K][K].
__global__ __launch_bounds__(256) void flip_damp_kernel(const double *__restrict__ H, int64_t ldh, int64_t K,
                                                        const double *__restrict__ lam, double *__restrict__ A) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= K * K) return;
    const int64_t i = idx / K, j = idx - i * K;
    double v = H[(K - 1 - i) * ldh + (K - 1 - j)];
    if (i == j) v += *lam;
    A[idx] = v;
}

// ---------------------------------------------------------------- blocked Cholesky (lower, in place)
// Diagonal block kb: factor the 32x32 block in LDS.
__global__ __launch_bounds__(256) void potrf_diag_kernel(double *__restrict__ A, int64_t K, int kb) {
    __shared__ double a[kNB][kNB + 1];
    const int tid = threadIdx.x;
    const int64_t o = (int64_t)kb * kNB;
    for (int e = tid; e < kNB * kNB; e += 256) a[e / kNB][e % kNB] = A[(o + e / kNB) * K + o + e % kNB];
    __syncthreads();
    for (int j = 0; j < kNB; ++j) {
        if (tid == 0) a[j][j] = sqrt(a[j][j]);
        __syncthreads();
        const double d = a[j][j];
        if (tid > j && tid < kNB) a[tid][j] /= d;
        __syncthreads();
        // trailing update of the block: a[i][k] -= a[i][j] a[k][j], j < k <= i
        for (int e = tid; e < kNB * kNB; e += 256) {
            const int i = e / kNB, k = e % kNB;
            if (k > j && i >= k) a[i][k] -= a[i][j] * a[k][j];
        }
        __syncthreads();
    }
    for (int e = tid; e < kNB * kNB; e += 256) {
        const int i = e / kNB, k = e % kNB;
        A[(o + i) * K + o + k] = k <= i ? a[i][k] : 0.0;
    }
}

// Panel below the diagonal block: rows r >= (kb+1)*32 of columns [kb*32, kb*32+32)
// solve X L^T = B (L the factored diagonal block): one thread per row.
__global__ __launch_bounds__(64) void trsm_panel_kernel(double *__restrict__ A, int64_t K, int kb) {
    __shared__ double L[kNB][kNB + 1];
    const int64_t o = (int64_t)kb * kNB;
    for (int e = threadIdx.x; e < kNB * kNB; e += 64) L[e / kNB][e % kNB] = A[(o + e / kNB) * K + o + e % kNB];
    __syncthreads();
    const int64_t r = o + kNB + (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (r >= K) return;
    double x[kNB];
#pragma unroll
    for (int j = 0; j < kNB; ++j) x[j] = A[r * K + o + j];
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
        double s = x[j];
#pragma unroll
        for (int k = 0; k < j; ++k) s -= x[k] * L[j][k];
        x[j] = s / L[j][j];
    }
#pragma unroll
    for (int j = 0; j < kNB; ++j) A[r * K + o + j] = x[j];
}

// Tiled fp64 update C[i][j] -= sum_{k<32} P[i][k] * Q[j][k] over a 64x64 tile per
// workgroup (each thread 4x4 outputs); P, Q, C row-major with the given strides.  Used
// for the Cholesky trailing update (lower tiles only).
__device__ __forceinline__ void tile_update(double *__restrict__ C, int64_t ldc, const double *__restrict__ P,
                                            int64_t ldp, const double *__restrict__ Q, int64_t ldq, int64_t m0,
                                            int64_t n0, int64_t mend, int64_t nend) {
    __shared__ double Ps[64][kNB + 1];
    __shared__ double Qs[64][kNB + 1];
    const int tid = threadIdx.x;
    for (int e = tid; e < 64 * kNB; e += 256) {
        const int rr = e / kNB, kk = e % kNB;
        Ps[rr][kk] = m0 + rr < mend ? P[(m0 + rr) * ldp + kk] : 0.0;
        Qs[rr][kk] = n0 + rr < nend ? Q[(n0 + rr) * ldq + kk] : 0.0;
    }
    __syncthreads();
    const int ti = (tid >> 4) * 4, tj = (tid & 15) * 4;
    double acc[4][4] = {};
#pragma unroll 8
    for (int k = 0; k < kNB; ++k) {
        double p[4], q[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            p[a] = Ps[ti + a][k];
            q[a] = Qs[tj + a][k];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = fma(p[a], q[b], acc[a][b]);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t i = m0 + ti + a, j = n0 + tj + b;
            if (i < mend && j < nend) C[i * ldc + j] -= acc[a][b];
        }
}

// Cholesky trailing update after panel kb: A[i][j] -= sum_k A[i][k] A[j][k] for
// i >= j >= (kb+1)*32 (tiles wholly above the diagonal are skipped).
__global__ __launch_bounds__(256) void syrk_kernel(double *__restrict__ A, int64_t K, int kb) {
    const int64_t base = (int64_t)(kb + 1) * kNB;
    const int64_t m0 = base + (int64_t)blockIdx.y * 64, n0 = base + (int64_t)blockIdx.x * 64;
    if (n0 > m0 + 63) return;
    const double *P = A + (int64_t)kb * kNB;  // column offset of the panel
    tile_update(A, K, P, K, P, K, m0, n0, K, K);
}

// ---------------------------------------------------------------- blocked lower-triangular inverse
// Cinv[ib][ib] = inverse of the 32x32 lower block C[ib][ib] (ib = workgroup): column j of
// the inverse by forward substitution (thread j).
__global__ __launch_bounds__(64) void trtri_diag_kernel(const double *__restrict__ C, double *__restrict__ Ci,
                                                        int64_t K) {
    __shared__ double L[kNB][kNB + 1];
    const int64_t o = (int64_t)blockIdx.x * kNB;
    for (int e = threadIdx.x; e < kNB * kNB; e += 64) L[e / kNB][e % kNB] = C[(o + e / kNB) * K + o + e % kNB];
    __syncthreads();
    const int j = threadIdx.x;
    if (j >= kNB) return;
    double x[kNB];
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
        double s = i == j ? 1.0 : 0.0;
#pragma unroll
        for (int k = 0; k < i; ++k) s -= L[i][k] * x[k];
        x[i] = i < j ? 0.0 : s / L[i][i];
    }
#pragma unroll
    for (int i = 0; i < kNB; ++i) Ci[(o + i) * K + o + j] = x[i];
}

// Column block jb of Cinv = C^-1 by block forward substitution (C X = E_jb):
//   X[ib][jb] = -Cinv[ib][ib] * sum_{kb=jb}^{ib-1} C[ib][kb] X[kb][jb],  ib = jb+1 .. nb-1,
// with X[jb][jb] = Cinv[jb][jb] from trtri_diag_kernel.  Column blocks are independent, so
// one launch runs all of them (workgroup jb), each reading C and only the blocks of its
// own column that it wrote itself; the 32x32x32 block products run on fp64 MFMA, each of
// the 4 waves computing one 16x16 quarter, with the next pair of tiles loaded into
// registers while the current pair is multiplied.
__global__ __launch_bounds__(256) void trtri_col_kernel(const double *__restrict__ C, double *__restrict__ Ci,
                                                        int64_t K, int nb) {
    __shared__ double As[kNB][kNB + 1];
    __shared__ double Bs[kNB][kNB + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t oj = (int64_t)blockIdx.x * kNB;
    const int wi = (wave >> 1) * 16, wj = (wave & 1) * 16;  // this wave's quarter of a tile
    const int lr = tid >> 3, lc = (tid & 7) * 4;             // tile loader: row, first of 4 columns
    // D layout of a 16x16 f64 MFMA tile: lane l, element r -> row l/16 + 4*r, column l%16
    const int dr = wi + (lane >> 4), dc = wj + (lane & 15);
    for (int ib = (int)blockIdx.x + 1; ib < nb; ++ib) {
        const int64_t oi = (int64_t)ib * kNB;
        v2f64 c0, c1, x0, x1;  // 4 consecutive doubles of a C tile row and of an X tile row
        auto load = [&](int kb) {
            const int64_t ok = (int64_t)kb * kNB;
            const v2f64 *pc = reinterpret_cast<const v2f64 *>(C + (oi + lr) * K + ok + lc);
            const v2f64 *px = reinterpret_cast<const v2f64 *>(Ci + (ok + lr) * K + oj + lc);
            c0 = pc[0];
            c1 = pc[1];
            x0 = px[0];
            x1 = px[1];
        };
        load((int)blockIdx.x);
        v4f64 acc = v4f64{0.0, 0.0, 0.0, 0.0};
        for (int kb = (int)blockIdx.x; kb < ib; ++kb) {
            __syncthreads();  // the previous products are done with As / Bs
            As[lr][lc] = c0.x;
            As[lr][lc + 1] = c0.y;
            As[lr][lc + 2] = c1.x;
            As[lr][lc + 3] = c1.y;
            Bs[lr][lc] = x0.x;
            Bs[lr][lc + 1] = x0.y;
            Bs[lr][lc + 2] = x1.x;
            Bs[lr][lc + 3] = x1.y;
            __syncthreads();
            if (kb + 1 < ib) load(kb + 1);
#pragma unroll
            for (int s = 0; s < kNB / 4; ++s) {
                const int k = 4 * s + (lane >> 4);
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64(As[wi + (lane & 15)][k], Bs[k][wj + (lane & 15)], acc, 0, 0,
                                                           0);
            }
        }
        // the sum to Bs, Cinv[ib][ib] to As, then X[ib][jb] = -Cinv[ib][ib] * sum
        const v2f64 *pd = reinterpret_cast<const v2f64 *>(Ci + (oi + lr) * K + oi + lc);
        const v2f64 d0 = pd[0], d1 = pd[1];
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 4; ++r) Bs[dr + 4 * r][dc] = acc[r];
        As[lr][lc] = d0.x;
        As[lr][lc + 1] = d0.y;
        As[lr][lc + 2] = d1.x;
        As[lr][lc + 3] = d1.y;
        __syncthreads();
        v4f64 out = v4f64{0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int s = 0; s < kNB / 4; ++s) {
            const int k = 4 * s + (lane >> 4);
            out = __builtin_amdgcn_mfma_f64_16x16x4f64(As[wi + (lane & 15)][k], Bs[k][wj + (lane & 15)], out, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Ci[(oi + dr + 4 * r) * K + oj + dc] = -out[r];
        // the block is read back (through memory) by this workgroup's later rows
        __threadfence();
    }
}

__global__ __launch_bounds__(256) void zero_upper_kernel(double *__restrict__ Ci, int64_t K) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= K * K) return;
    const int64_t i = idx / K, j = idx - i * K;
    if (j > i) Ci[idx] = 0.0;
}

// U = J Cinv J (upper), written with leading dimension ldu.
__global__ __launch_bounds__(256) void flip_kernel(const double *__restrict__ Ci, int64_t K, double *__restrict__ U,
                                                   int64_t ldu) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= K * K) return;
    const int64_t i = idx / K, j = idx - i * K;
    U[i * ldu + j] = Ci[(K - 1 - i) * K + (K - 1 - j)];
}

// ---------------------------------------------------------------- column loop
__global__ __launch_bounds__(256) void widen_kernel(const uint16_t *__restrict__ W, int64_t ldw, int64_t R, int64_t K,
                                                    double *__restrict__ Wd) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= R * K) return;
    const int64_t r = idx / K, c = idx - r * K;
    Wd[idx] = bf16_to_f64(W[r * ldw + c]);
}

// One 32-column block (one mask word) of every row: selection at group starts,
// compensation inside the block, mask word + 16 kept values (bf16) + 32 errors out.
// One thread per row; the block's weights and the group's saliencies live in
// per-thread LDS slots (33-double stride, so the threads of a wave spread over the
// banks), which keeps the sequential column loop free of register spills.
constexpr int kBlkThreads = 64;

template <int M>
__global__ __launch_bounds__(kBlkThreads) void sgpt_block_kernel(const double *__restrict__ Wd, int64_t R, int64_t K,
                                                                 const double *__restrict__ U, int64_t ldu, int64_t c0,
                                                                 double *__restrict__ Err,
                                                                 uint32_t *__restrict__ masks,
                                                                 uint16_t *__restrict__ values) {
    constexpr int N = M / 2;
    __shared__ double Ub[kNB][kNB + 1];
    __shared__ double wsl[kBlkThreads][kNB + 1];
    __shared__ double ssl[kBlkThreads][kNB + 1];
    for (int e = threadIdx.x; e < kNB * kNB; e += kBlkThreads)
        Ub[e / kNB][e % kNB] = U[(c0 + e / kNB) * ldu + c0 + e % kNB];
    __syncthreads();
    const int64_t r = (int64_t)blockIdx.x * kBlkThreads + threadIdx.x;
    if (r >= R) return;
    double *w = wsl[threadIdx.x];
    double *sal = ssl[threadIdx.x];
    for (int a = 0; a < kNB; ++a) w[a] = Wd[r * K + c0 + a];
    uint32_t keep = 0;
    for (int a = 0; a < kNB; ++a) {
        if (a % M == 0) {
            // saliency w^2 / U[c][c]^2 of the group's columns; keep the N largest
            // (ties: lower column), by counting the columns that come first
            for (int c = 0; c < M; ++c) {
                const double dc = Ub[a + c][a + c];
                sal[c] = (w[a + c] * w[a + c]) / (dc * dc);
            }
            for (int c = 0; c < M; ++c) {
                const double sc = sal[c];
                int ahead = 0;
                for (int c2 = 0; c2 < M; ++c2)
                    ahead += (c2 != c && (sal[c2] > sc || (sal[c2] == sc && c2 < c))) ? 1 : 0;
                keep |= (ahead < N ? 1u : 0u) << (a + c);
            }
        }
        const bool kept = (keep >> a) & 1u;
        const double e = kept ? 0.0 : w[a] / Ub[a][a];
        if (!kept) {
            w[a] = 0.0;
            for (int a2 = a + 1; a2 < kNB; ++a2) w[a2] = fma(-e, Ub[a][a2], w[a2]);
        }
        Err[r * kLB + c0 % kLB + a] = e;
    }
    const int64_t word = c0 / kNB;
    masks[r * (K / kNB) + word] = keep;
    uint32_t out[8];
    uint32_t mm = keep;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int ca = low_bit(mm);  // stays in the slot for any mask
        mm &= mm - 1;
        const int cb = low_bit(mm);
        mm &= mm - 1;
        out[t] = (uint32_t)f64_to_bf16_rne(w[ca]) | ((uint32_t)f64_to_bf16_rne(w[cb]) << 16);
    }
    uint4 *v4 = reinterpret_cast<uint4 *>(values + r * (K / 2) + 16 * word);
    v4[0] = make_uint4(out[0], out[1], out[2], out[3]);
    v4[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

// Compensation of later columns: Wd[r][n0 + j] -= sum_k Err[r][e0 + k] * U[u0 + k][n0 + j]
// for r < R, j < ncols, k < kw (kw a multiple of 16).  On the fp64 matrix cores: a 64x64
// tile of Wd per workgroup (4 waves, 32x32 each = 2x2 MFMA tiles), 16 k per LDS stage.
__global__ __launch_bounds__(256) void sgpt_update_kernel(double *__restrict__ Wd, int64_t R, int64_t K, int64_t n0,
                                                          int64_t ncols, const double *__restrict__ Err, int e0,
                                                          const double *__restrict__ U, int64_t ldu, int64_t u0,
                                                          int kw) {
    __shared__ double As[16][64];  // As[k][m] = Err[m0 + m][e0 + k0 + k]
    __shared__ double Bs[16][64];  // Bs[k][n] = U[u0 + k0 + k][n0 + nb0 + n]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * 64, nb0 = (int64_t)blockIdx.x * 64;
    const int wi = (wave >> 1) * 32, wj = (wave & 1) * 32;
    v4f64 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = v4f64{0.0, 0.0, 0.0, 0.0};
    for (int k0 = 0; k0 < kw; k0 += 16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = tid + 256 * e;
            const int m = idx >> 4, k = idx & 15;  // 16 consecutive k of one row of Err per 16 threads
            As[k][m] = m0 + m < R ? Err[(m0 + m) * kLB + e0 + k0 + k] : 0.0;
            const int kb = idx >> 6, n = idx & 63;  // one row of U, 64 consecutive columns
            Bs[kb][n] = nb0 + n < ncols ? U[(u0 + k0 + kb) * ldu + n0 + nb0 + n] : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int tk = 4 * st + (lane >> 4);
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const double av = As[tk][wi + 16 * a + (lane & 15)];
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const double bv = Bs[tk][wj + 16 * b + (lane & 15)];
                    acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[a][b], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }
    // D layout of the 16x16 f64 tile: lane l, element r -> row l/16 + 4*r, column l%16
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t i = m0 + wi + 16 * a + (lane >> 4) + 4 * r;
                const int64_t j = nb0 + wj + 16 * b + (lane & 15);
                if (i < R && j < ncols) Wd[i * K + n0 + j] -= acc[a][b][r];
            }
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

// Workspace layout (bytes): [A/U: K*K fp64][Cinv: K*K fp64][lambda: 32 fp64][Wd: R*K fp64][Err: R*128 fp64]
size_t sparsegpt_factor_workspace(int64_t K) { return (size_t)(2 * K * K + 32) * sizeof(double); }

size_t sparsegpt_workspace(int64_t R, int64_t K) {
    return sparsegpt_factor_workspace(K) + (size_t)(R * K + R * kLB) * sizeof(double);
}

hipError_t launch_hessian(const uint16_t *X, int64_t T, int64_t K, int64_t ldx, double *H, int64_t ldh,
                          hipStream_t st) {
    const int g = (int)((K + kHT - 1) / kHT);
    const unsigned tiles = (unsigned)((int64_t)g * (g + 1) / 2);  // on and above the diagonal
    hipLaunchKernelGGL(hessian_kernel, dim3(tiles), dim3(256), 0, st, X, T, K, ldx, H, ldh, g);
    return hipGetLastError();
}

// U (upper, ldu) with U^T U = (H + lambda I)^-1; ws: sparsegpt_factor_workspace(K) bytes.
hipError_t launch_inverse_factor(const double *H, int64_t ldh, int64_t K, double damp, double *U, int64_t ldu,
                                 void *ws, hipStream_t st) {
    double *A = (double *)ws;
    double *Ci = A + K * K;
    double *lam = Ci + K * K;
    hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(256), 0, st, H, ldh, K, damp, lam);
    hipLaunchKernelGGL(flip_damp_kernel, dim3(blocks_for(K * K)), dim3(256), 0, st, H, ldh, K, lam, A);
    const int nb = (int)(K / kNB);
    for (int kb = 0; kb < nb; ++kb) {
        hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(256), 0, st, A, K, kb);
        if (kb + 1 < nb) {
            const int64_t rest = K - (int64_t)(kb + 1) * kNB;
            hipLaunchKernelGGL(trsm_panel_kernel, dim3((unsigned)((rest + 63) / 64)), dim3(64), 0, st, A, K, kb);
            const unsigned t = (unsigned)((rest + 63) / 64);
            hipLaunchKernelGGL(syrk_kernel, dim3(t, t), dim3(256), 0, st, A, K, kb);
        }
    }
    hipLaunchKernelGGL(zero_upper_kernel, dim3(blocks_for(K * K)), dim3(256), 0, st, Ci, K);
    hipLaunchKernelGGL(trtri_diag_kernel, dim3((unsigned)nb), dim3(64), 0, st, A, Ci, K);
    hipLaunchKernelGGL(trtri_col_kernel, dim3((unsigned)nb), dim3(256), 0, st, A, Ci, K, nb);
    hipLaunchKernelGGL(flip_kernel, dim3(blocks_for(K * K)), dim3(256), 0, st, Ci, K, U, ldu);
    return hipGetLastError();
}

hipError_t launch_sparsegpt(const uint16_t *W, int64_t ldw, int64_t R, int64_t K, const double *H, int64_t ldh,
                            int N, int M, double damp, uint32_t *masks, uint16_t *values, void *ws, hipStream_t st) {
    (void)N;  // N == M/2 is checked by the caller
    double *A = (double *)ws;           // becomes U
    double *Wd = A + 2 * K * K + 32;
    double *Err = Wd + R * K;
    hipError_t e = launch_inverse_factor(H, ldh, K, damp, A, K, ws, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(widen_kernel, dim3(blocks_for(R * K)), dim3(256), 0, st, W, ldw, R, K, Wd);
    // Column blocks of 32 in lazy batches of 128: a block's errors compensate the rest of its
    // batch at once; a batch's errors compensate every later column in one rank-128 update.
    auto update = [&](int64_t n0, int64_t ncols, int e0, int64_t u0, int kw) {
        hipLaunchKernelGGL(sgpt_update_kernel, dim3((unsigned)((ncols + 63) / 64), (unsigned)((R + 63) / 64)),
                           dim3(256), 0, st, Wd, R, K, n0, ncols, Err, e0, A, K, u0, kw);
    };
    for (int64_t b0 = 0; b0 < K; b0 += kLB) {
        const int64_t b1 = b0 + kLB < K ? b0 + kLB : K;
        for (int64_t c0 = b0; c0 < b1; c0 += kNB) {
            const unsigned g = (unsigned)((R + kBlkThreads - 1) / kBlkThreads);
            switch (M) {
            case 4: hipLaunchKernelGGL(sgpt_block_kernel<4>, dim3(g), dim3(kBlkThreads), 0, st, Wd, R, K, A, K, c0, Err, masks, values); break;
            case 8: hipLaunchKernelGGL(sgpt_block_kernel<8>, dim3(g), dim3(kBlkThreads), 0, st, Wd, R, K, A, K, c0, Err, masks, values); break;
            case 16: hipLaunchKernelGGL(sgpt_block_kernel<16>, dim3(g), dim3(kBlkThreads), 0, st, Wd, R, K, A, K, c0, Err, masks, values); break;
            case 32: hipLaunchKernelGGL(sgpt_block_kernel<32>, dim3(g), dim3(kBlkThreads), 0, st, Wd, R, K, A, K, c0, Err, masks, values); break;
            default: return hipErrorInvalidValue;
            }
            if (c0 + kNB < b1) update(c0 + kNB, b1 - c0 - kNB, (int)(c0 - b0), c0, kNB);
        }
        if (b1 < K) update(b1, K - b1, 0, b0, (int)(b1 - b0));
    }
    return hipGetLastError();
}

}  // namespace nmk
