// nm_spmv_common.h -- pieces shared by the sparse matrix-vector kernels (N:M with any
// metadata format, and 50% unstructured rows): the LDS layout of x and its staging, and
// the pair-of-kept-weights dot product.  Internal; included by .hip files only.
#pragma once

#include "nm_device.h"
#include "nm_kernels.h"

namespace nmk {
namespace {

// Blocked LDS layout of x (the one-token word walk, and the unstructured kernel at every
// B).  B = 1: each 32-column block is 16 dwords of bf16 pairs plus one pad dword (17
// dwords), so lanes walking different words spread over the banks.  B > 1: tokens are
// interleaved per column -- column c holds S bf16 (S = B rounded up to 2, 4 or 8,
// zero-filled) -- so one 4/8/16-byte LDS load gathers a column for every token; blocks
// are 16*S dwords plus S/2 pad dwords (keeping 8/16-byte alignment).
template <int B>
struct XLayout {
    static constexpr int S = B == 1 ? 1 : (B <= 2 ? 2 : (B <= 4 ? 4 : 8));
    static constexpr int kBlk = B == 1 ? 17 : 16 * S + S / 2;  // dwords per 32-column block
};

constexpr int blk_dwords(int B) {
    return B == 1 ? 17 : (B <= 2 ? 33 : (B <= 4 ? 66 : 132));
}

// Panel LDS layout of x (the N:M word walk at B >= 2).  Columns hold the same S
// interleaved token slots (S/2 dwords), but a block's 32 columns are stacked at a stride
// of 64 dwords: a panel is 32 rows of 64 dwords, and the 128/S blocks side by side in it
// each own one stripe of S/2 dwords of every row.  In the word walk lane 2i walks word i
// of its 64-word strip and lane 2i+1 word 32+i; block j of a strip goes to the panel and
// stripe of that lane, L = 2j (j < 32) or 2j - 63, so every lane gathers from LDS banks
// that no other lane of its group of 128/S lanes touches, whatever columns the masks
// pick (the blocked layout puts the columns of different lanes' words on shared banks at
// random: about half the LDS cycles of the walk went to bank conflicts at 2-4 tokens).
// A 64-word strip takes S/2 panels (64*S bytes per word); the layout is defined for
// every word index, so a lane may gather from any block.
template <int B>
struct XPanel {
    static constexpr int S = XLayout<B>::S;
    static constexpr int kColDw = S / 2;           // dwords per column (the token slots)
    static constexpr int kGroup = 128 / S;         // blocks side by side in one panel
    static constexpr int kRowDw = 64;              // dwords per panel row (column stride)
    static constexpr int kPanelDw = 32 * kRowDw;   // dwords per panel
    static constexpr int kWordBytes = 64 * S;      // LDS bytes per word, in whole strips
};

// Dword offset of column 0 of block w (w counted from the slice start) in the panel layout.
template <int B>
__device__ __forceinline__ int panel_block(int w) {
    using P = XPanel<B>;
    const int j = w & 63, L = j < 32 ? 2 * j : 2 * j - 63;
    return ((w >> 6) * P::kColDw + L / P::kGroup) * P::kPanelDw + (L % P::kGroup) * P::kColDw;
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Gather of one column for the S token slots (S/2 dwords: token pairs); CS is the
// column stride in dwords (S/2 in the blocked layout, 64 in the panel layout).
template <int S, int CS>
__device__ __forceinline__ void gather_col(const uint32_t *blk, int c, uint32_t (&d)[S / 2]) {
    if constexpr (S == 2) {
        d[0] = blk[CS * c];
    } else if constexpr (S == 4) {
        const u32x2 t = *reinterpret_cast<const u32x2 *>(blk + CS * c);
        d[0] = t.x;
        d[1] = t.y;
    } else {
        const u32x4 t = *reinterpret_cast<const u32x4 *>(blk + CS * c);
        d[0] = t.x;
        d[1] = t.y;
        d[2] = t.z;
        d[3] = t.w;
    }
}

// One pair of kept weights: the inputs of columns c0 and c1 of the word's block (per
// token) meet the packed value pair v in one v_dot2_f32_bf16.  PANEL: blk is the block's
// column 0 in the panel layout (B >= 2), else in the blocked layout.
template <int B, bool PANEL = false>
__device__ __forceinline__ void dot_pair(uint32_t v, const uint32_t *blk, int c0, int c1, float (&acc)[B]) {
    constexpr int S = XLayout<B>::S;
    static_assert(!PANEL || S > 1, "the panel layout holds two or more token slots");
    constexpr int CS = PANEL ? XPanel<B>::kRowDw : S / 2;
    if constexpr (S == 1) {
        const uint16_t *xw = reinterpret_cast<const uint16_t *>(blk);
        const uint32_t pr = (uint32_t)xw[c0] | ((uint32_t)xw[c1] << 16);
        acc[0] = dot2_bf16(v, pr, acc[0]);
    } else {
        uint32_t d0[S / 2], d1[S / 2];
        gather_col<S, CS>(blk, c0, d0);
        gather_col<S, CS>(blk, c1, d1);
#pragma unroll
        for (int j = 0; j < S / 2; ++j) {
            // (token 2j of column c0, token 2j of column c1), then the same for 2j+1
            if (2 * j < B) acc[2 * j] = dot2_bf16(v, __builtin_amdgcn_perm(d1[j], d0[j], 0x05040100u), acc[2 * j]);
            if (2 * j + 1 < B)
                acc[2 * j + 1] = dot2_bf16(v, __builtin_amdgcn_perm(d1[j], d0[j], 0x07060302u), acc[2 * j + 1]);
        }
    }
}

// The same at one token, with the two columns given by their LDS byte addresses.
__device__ __forceinline__ void dot_pair_at(uint32_t v, const uint8_t *p0, const uint8_t *p1, float &acc) {
    const uint32_t pr = (uint32_t)*reinterpret_cast<const uint16_t *>(p0) |
                        ((uint32_t)*reinterpret_cast<const uint16_t *>(p1) << 16);
    acc = dot2_bf16(v, pr, acc);
}

// Matrix of the set that owns global row r (0 <= r < R).  The launcher pads row0 past
// the last matrix with the total row count, so p counts the bounds row0[q] <= r.  The
// test is the sign of row0[q] - 1 - r (no overflow for 0 <= r, row0[q] <= INT_MAX),
// which keeps it in scalar integer arithmetic: a boolean compare is materialised
// through a vector register here, and reusing that register makes the wave wait for
// its in-flight loads.
__device__ __forceinline__ int owner(const SpmvSet &set, int r) {
    int p = 0;
#pragma unroll
    for (int q = 1; q < kMaxMats; ++q) p += (int)((uint32_t)(set.row0[q] - 1 - r) >> 31);
    return p;
}

// Stages columns [32*w0, 32*(w0+nws)) of x (B tokens, row stride ldx) into LDS in the
// blocked layout, or in the panel layout (PANEL, B >= 2), all NT threads of the workgroup
// taking part; first_round() runs once, right after the first round of x loads has been
// issued (callers put their first weight loads there).  The caller synchronises the
// workgroup afterwards.
template <int B, int NT, bool PANEL = false, class F>
__device__ __forceinline__ void stage_x(uint32_t *xs, const uint16_t *__restrict__ x, int64_t ldx, int w0, int nws,
                                        F &&first_round) {
    static_assert(!PANEL || XLayout<B>::S > 1, "the panel layout holds two or more token slots");
    if constexpr (XLayout<B>::S == 1) {
        // 16-byte loads; 8 bf16 per chunk, 4 chunks per 32-column block.  No load sits under
        // a lane condition: the part of a round beyond the slice is skipped by a uniform
        // test, and a thread whose chunk lies past the slice loads the slice's last chunk
        // again (and stores nothing).  Each loaded register is then consumed by an empty
        // asm statement outside the store's lane condition.  Otherwise the compiler is left
        // unsure whether an x load is still in flight, and it waits for every load -- the
        // first weight batch included -- before the next batch's loads go out: a memory
        // round trip per wave.
        constexpr int kStage = 4;
        const int chunks = nws * 4;
        const u32x4 *xc = reinterpret_cast<const u32x4 *>(x + (int64_t)w0 * 32);
        for (int i0 = 0; i0 < chunks || i0 == 0; i0 += NT * kStage) {
            u32x4 r[kStage];
#pragma unroll
            for (int j = 0; j < kStage; ++j) {
                if (j > 0 && i0 + j * NT >= chunks) break;
                r[j] = xc[min(i0 + j * NT + (int)threadIdx.x, chunks - 1)];
            }
            if (i0 == 0) first_round();
#pragma unroll
            for (int j = 0; j < kStage; ++j) {
                if (j > 0 && i0 + j * NT >= chunks) break;
                const int i = i0 + j * NT + (int)threadIdx.x;
                if (i < chunks) {
                    uint32_t *d = xs + (i >> 2) * XLayout<B>::kBlk + (i & 3) * 4;
                    d[0] = r[j].x;
                    d[1] = r[j].y;
                    d[2] = r[j].z;
                    d[3] = r[j].w;
                }
                asm volatile("" ::"v"(r[j].x), "v"(r[j].y), "v"(r[j].z), "v"(r[j].w));
            }
        }
    } else {
        // Eight columns per thread and round: one 16-byte load of every token, transposed
        // with byte permutes into the interleaved per-column layout (the eight columns'
        // 4*S dwords are contiguous in LDS: S 16-byte stores).  The loads are
        // unconditional (a thread past the slice re-reads its last eight columns) and the
        // parts of a round beyond the slice are skipped by a uniform test: loads under a
        // lane condition were issued one or two at a time, each waiting for the previous.
        constexpr int S = XLayout<B>::S;
        constexpr int kStage = 8 / S;  // 8 x 16-byte loads in flight per thread and round
        const int octs = nws * 4;
        const int rounds = (octs + NT - 1) / NT;  // loads per thread and token (uniform)
        const uint16_t *xw = x + (int64_t)w0 * 32;
        for (int i0 = 0; i0 < octs || i0 == 0; i0 += NT * kStage) {
            const int left = rounds - i0 / NT;
            u32x4 r[kStage][S];
#pragma unroll
            for (int j = 0; j < kStage; ++j) {
                if (j > 0 && j >= left) break;
                const int i = min(i0 + j * NT + (int)threadIdx.x, octs - 1);
#pragma unroll
                for (int b = 0; b < S; ++b)
                    r[j][b] = b < B ? *reinterpret_cast<const u32x4 *>(xw + (int64_t)b * ldx + 8 * i)
                                    : u32x4{0u, 0u, 0u, 0u};
            }
            if (i0 == 0) first_round();
#pragma unroll
            for (int j = 0; j < kStage; ++j) {
                if (j > 0 && j >= left) break;
                const int i = min(i0 + j * NT + (int)threadIdx.x, octs - 1);
                {
                    const int c = 8 * i;  // first column of the eight, within the slice
                    uint32_t col[4 * S];  // column c+k: dwords k*S/2 .. k*S/2 + S/2 - 1
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
#pragma unroll
                        for (int t = 0; t < S / 2; ++t) {
                            col[(2 * q) * (S / 2) + t] = __builtin_amdgcn_perm(r[j][2 * t + 1][q], r[j][2 * t][q], 0x05040100u);
                            col[(2 * q + 1) * (S / 2) + t] =
                                __builtin_amdgcn_perm(r[j][2 * t + 1][q], r[j][2 * t][q], 0x07060302u);
                        }
                    }
                    if constexpr (PANEL) {
                        // eight columns of one block: one S/2-dword store per column, 64 dwords apart
                        uint32_t *d = xs + panel_block<B>(c >> 5) + (c & 31) * XPanel<B>::kRowDw;
#pragma unroll
                        for (int k = 0; k < 8; ++k) {
                            if constexpr (S == 2) {
                                d[k * XPanel<B>::kRowDw] = col[k];
                            } else if constexpr (S == 4) {
                                *reinterpret_cast<u32x2 *>(d + k * XPanel<B>::kRowDw) = u32x2{col[2 * k], col[2 * k + 1]};
                            } else {
                                *reinterpret_cast<u32x4 *>(d + k * XPanel<B>::kRowDw) =
                                    u32x4{col[4 * k], col[4 * k + 1], col[4 * k + 2], col[4 * k + 3]};
                            }
                        }
                    } else {
                        u32x4 *d = reinterpret_cast<u32x4 *>(xs + (c >> 5) * XLayout<B>::kBlk + (c & 31) * (S / 2));
#pragma unroll
                        for (int v = 0; v < S; ++v) d[v] = u32x4{col[4 * v], col[4 * v + 1], col[4 * v + 2], col[4 * v + 3]};
                    }
                }
            }
        }
    }
}

}  // namespace
}  // namespace nmk
