// nm_spmv_tile.hip -- N:M sparse matrix times a small batch of input vectors (5..8 tokens,
// and 3..4 on rows too wide for the other kernel's LDS) with the products on the matrix
// cores of gfx950.
//
// What it computes: the same product as nm_spmv.hip, over the same packed operands --
// one 32-bit mask word per 32 columns whose set bits pair, in increasing column order,
// with the stored values ("SparseDecoding: Decoding-Aware Pruning ..." (ai.info summary),
// Methodology Steps 2-3; "SparseDecoding:解码感知的准确高效大模型剪枝框架"
// (paper.rainbus.top), 方法步骤详情 第四步) -- for B = 5..8 input vectors, and for B = 3..4
// where a row's x no longer fits the word-per-lane kernel's LDS slice (K > 10240).
//
// Why a second kernel: with one lane per mask word, every kept weight costs a gather of
// its input column for all B tokens from LDS (16 bytes at B = 8, at a data-dependent
// column, so the lanes of a wave collide on LDS banks) plus B/2 byte permutes and B/2
// packed dot products; at B = 8 that ALU and LDS work, not HBM, bounds the launch.  Here
// the walk over a word stays the fixed 16 steps (lowest set bit -> column, clear it), but
// each step writes the kept value into a dense 16-row tile in LDS instead of reading x;
// the tile times the B input vectors is then one 16x32x16 bf16 product per word column
// on the matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation), whose input operand
// holds tokens 0..B-1 in its first B lanes of each row group and zeros in the others.
//
// Layout of the work:
//   * a workgroup (8 or 16 waves) owns a unit of 16-row tiles at a time; its steps of
//     4 words go round-robin to the waves (wave w: steps w, w + W, ...), one word per lane;
//   * tile rows 0-7 and 8-15 are 8 consecutive rows of one matrix each (plain launch:
//     the same matrix; gated MLP: gate rows i..i+7, then up rows i..i+7);
//   * a step loads 128 bytes of values per row (two 16-byte loads per lane, rows 0-7
//     then rows 8-15, 8 lanes per row, contiguous), the lane's mask word of both row
//     halves, and the step's 4 x 32 columns of x straight into the MFMA operand
//     registers (x is re-read by every tile: an L2 hit -- except where every wave has
//     exactly four steps per unit, K = 4096 with 8 waves or 8192 with 16: a wave's x
//     columns are then the same in every unit and stay in registers after its first);
//     a swap of 16-byte halves between lane pairs gives each lane the 16 values of its
//     word, as in nm_spmv.hip;
//   * the lane zeroes its word's 32 columns of the wave's dense tile and writes its 16
//     kept values at their columns; four MFMAs then add the step into the wave's 16xB
//     accumulator (lane l: rows 4*(l/16)..+3 of token l%16);
//   * at the end of a unit the W waves' partial sums meet in LDS and are added in wave
//     order (deterministic), then rounded once to bf16 -- for the gated MLP combined
//     first as silu(gate) * up.
// Every load goes through a raw buffer descriptor whose base carries the step's column
// offset and whose size ends at the last valid row, so rows past the matrix, token lanes
// past B and the one batch issued past the end of the work read zeros without touching
// memory, and every wave issues the same loads in the same order.
#include <atomic>

#include "nm_device.h"
#include "nm_kernels.h"
#include "nm_spmv_common.h"

namespace nmk {
namespace {

constexpr int kTRows = 16;                        // rows per MFMA tile (the MFMA's M)
constexpr int kTStep = 4;                         // words per row and step
constexpr int kTRowBytes = 16 + kTStep * 64;      // tile row: 16-byte lead pad + 4 x 32 bf16
constexpr int kTWaveBytes = kTRows * kTRowBytes + 16;  // one wave's dense tile + a 16-byte tail pad
constexpr uint32_t kXOut = 0x40000000u;           // x offset of token lanes >= B: past the buffer

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// LDS of a workgroup of W waves walking TT tiles per step: the waves' dense tiles, then
// two buffers of the waves' partial sums ([W][B][16*TT] floats each).
template <int B, int TT, int W>
constexpr size_t tile_lds_bytes() {
    return (size_t)W * kTWaveBytes + 2 * (size_t)W * B * kTRows * TT * 4;
}

// One step's loads: 4 words of each of the 16 rows of each of the TT tiles.
template <int TT>
struct TBatch {
    u32x4 va[TT], vb[TT];  // 16-byte value chunk (lane & 7) of tile row (lane >> 3), of row 8 + (lane >> 3)
    uint32_t ma[TT], mb[TT];  // mask word ((lane & 7) >> 1) of the same two rows
    u32x4 xp[kTStep / 2];     // x of word columns 2p (lanes n < 8) and 2p+1 (lanes n >= 8), shared by the tiles
};

// Where a unit's rows live (8-row quarters: tile t has quarters 2t and 2t+1), and where
// its outputs go.
template <int TT>
struct TileRows {
    const uint8_t *m[2 * TT];  // masks of the first row of each quarter
    const uint8_t *v[2 * TT];  // values of the first row of each quarter
    int valid[2 * TT];         // rows of each quarter inside the matrix (0..8)
    int p;                     // output matrix
    int local;                 // first output row of the unit within matrix p
    int rows;                  // rows of matrix p (plain launch) / of the gate matrix (gated MLP)
};

// Rows of unit u.  Plain launch: 16*TT consecutive rows of one matrix.  Gated MLP: gate
// and up rows i0..i0+8*TT-1; tile t holds gate rows i0+8t..+7 in rows 0-7 and the same
// up rows in rows 8-15.
template <int EPI, int TT>
__device__ __forceinline__ TileRows<TT> tile_rows(const SpmvSet &set, int unit, int KW) {
    TileRows<TT> t;
    if constexpr (EPI == kEpiSwiGLU) {
        const int i0 = unit * 8 * TT;
#pragma unroll
        for (int q = 0; q < 2 * TT; ++q) {
            const int r = i0 + 8 * (q >> 1);
            t.m[q] = static_cast<const uint8_t *>(set.meta[q & 1]) + (int64_t)r * KW * 4;
            t.v[q] = reinterpret_cast<const uint8_t *>(set.values[q & 1]) + (int64_t)r * KW * 32;
            t.valid[q] = min(max(set.row0[1] - r, 0), 8);
        }
        t.p = 0;
        t.local = i0;
        t.rows = set.row0[1];
    } else {
        const int tb = unit * kTRows * TT;
        const int p = owner(set, tb);  // a unit never straddles two matrices
        const int lb = tb - set.row0[p];
        const int rp = set.row0[p + 1] - set.row0[p];
#pragma unroll
        for (int q = 0; q < 2 * TT; ++q) {
            t.m[q] = static_cast<const uint8_t *>(set.meta[p]) + (int64_t)(lb + 8 * q) * KW * 4;
            t.v[q] = reinterpret_cast<const uint8_t *>(set.values[p]) + (int64_t)(lb + 8 * q) * KW * 32;
            t.valid[q] = min(max(rp - lb - 8 * q, 0), 8);
        }
        t.p = p;
        t.local = lb;
        t.rows = rp;
    }
    return t;
}

// Loads of one step at word column cw (live = false: the same loads with empty ranges);
// LX = false leaves out the x operand (kept in registers by the caller).
template <int B, int TT, bool LX = true>
__device__ __forceinline__ void load_tbatch(TBatch<TT> &bt, const TileRows<TT> &tr, int cw, int KW,
                                            const uint16_t *x, int64_t ldx, uint32_t vo, uint32_t mo, uint32_t xo,
                                            bool live) {
    const int64_t vrow = (int64_t)KW * 32, mrow = (int64_t)KW * 4;
#pragma unroll
    for (int q = 0; q < 2 * TT; ++q) {
        const int64_t vn = live ? tr.valid[q] * vrow - (int64_t)cw * 32 : 0;
        const int64_t mn = live ? tr.valid[q] * mrow - (int64_t)cw * 4 : 0;
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(tr.v[q] + (int64_t)cw * 32, vn > 0 ? vn : 0);
        const __amdgpu_buffer_rsrc_t rm = make_rsrc(tr.m[q] + (int64_t)cw * 4, mn > 0 ? mn : 0);
        // (the 16 bytes of masks per row and step are a part of a line the next steps
        // read again: a default load keeps the line in the caches for them)
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rv, vo, 0, kLoadNT);
        const uint32_t m = __builtin_amdgcn_raw_buffer_load_b32(rm, mo, 0, 0);
        if (q & 1) {
            bt.vb[q >> 1] = v;
            bt.mb[q >> 1] = m;
        } else {
            bt.va[q >> 1] = v;
            bt.ma[q >> 1] = m;
        }
    }
    if constexpr (LX) {
        const int64_t xn = live ? (int64_t)(B - 1) * ldx * 2 + (int64_t)(KW - cw) * 64 : 0;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (int64_t)cw * 32, xn);
#pragma unroll
        for (int j = 0; j < kTStep / 2; ++j) bt.xp[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo + j * 128u, 0, 0);
    }
}

// Swap one dword with the neighbouring lane of the pair (lane ^ 1).
__device__ __forceinline__ uint32_t tpair_swap(uint32_t v) {
    // every lane has a source lane: "old" is never read (v itself: no zeroed register)
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false);  // quad_perm(1,0,3,2)
}

// One tile of one step: expand the lane's word into the wave's dense tile, then four MFMAs.
//
// Lane l's word: row (l & 1) * 8 + (l >> 3) of the tile, word column (l & 7) >> 1.  Its
// 32 columns are zeroed and its 16 kept values written at their columns.  Even lanes
// walk the word from its lowest set bit up, odd lanes from its highest set bit down (the
// lowest set bit of the bit-reversed mask, the values taken in reverse order): at each
// of the 16 steps the lanes then write near opposite ends of their words, which spreads
// the writes of lanes whose words start on the same LDS bank.  A word without exactly 16
// set bits (rows past the matrix, whose loads read zero, or a malformed mask) walks the
// mask 0xFFFF instead, so every one of the 16 bit scans has a set bit to find and the
// writes stay inside the lane's own word.  The zeroing writes of lanes with rows 8..15 take
// the word's 16-byte chunks in the order 2, 3, 0, 1, so the 16 lanes of each group of a
// 16-byte write cover distinct banks.  The wave's LDS operations execute in issue order,
// so the expansion is complete before the operand reads that follow it, and the operand
// reads of one tile before the expansion of the next tile into the same LDS.
__device__ __forceinline__ void walk_tile(const u32x4 &va, const u32x4 &vb, uint32_t ma, uint32_t mb,
                                          const u32x4 (&xq)[kTStep], uint8_t *tw, int lane, f32x4 &acc) {
    const bool odd = lane & 1;
    const uint32_t s_x = odd ? va.x : vb.x, s_y = odd ? va.y : vb.y;
    const uint32_t s_z = odd ? va.z : vb.z, s_w = odd ? va.w : vb.w;
    const uint32_t r_x = tpair_swap(s_x), r_y = tpair_swap(s_y), r_z = tpair_swap(s_z), r_w = tpair_swap(s_w);
    // the word's 16 values in walk order: even lanes ascending, odd lanes descending
    // (dword d of the odd lane = the two values of dword 7 - d, halves swapped); one byte
    // permute per dword picks the lane's dword and, on odd lanes, swaps its halves
    const uint32_t od[8] = {vb.w, vb.z, vb.y, vb.x, r_w, r_z, r_y, r_x};
    const uint32_t ev[8] = {va.x, va.y, va.z, va.w, r_x, r_y, r_z, r_w};
    const uint32_t sel = odd ? 0x05040706u : 0x03020100u;  // odd: od[d] halves swapped; even: ev[d]
    uint32_t v[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) v[d] = __builtin_amdgcn_perm(od[d], ev[d], sel);
    uint32_t m = odd ? __builtin_bitreverse32(mb) : ma;
    m = __builtin_popcount(m) == 16 ? m : 0xFFFFu;
    uint8_t *ub = tw + ((lane & 1) * 8 + (lane >> 3)) * kTRowBytes + 16 + ((lane & 7) >> 1) * 64;
    uint8_t *wb = odd ? ub + 62 : ub;  // column c of the walk order sits at wb + step * c
    const int step = odd ? -2 : 2;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4 *>(ub + 16 * ((k + 2 * (lane & 1)) & 3)) = zero;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const int c = __builtin_ctz(m);
        m &= m - 1;
        const uint16_t val = (t & 1) ? (uint16_t)(v[t >> 1] >> 16) : (uint16_t)v[t >> 1];
        *reinterpret_cast<uint16_t *>(wb + step * c) = val;
    }
    __builtin_amdgcn_wave_barrier();
    const uint8_t *ar = tw + (lane & 15) * kTRowBytes + 16 + (lane >> 4) * 16;
#pragma unroll
    for (int j = 0; j < kTStep; ++j) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(ar + 64 * j);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, xq[j]),
                                                      acc, 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
}

// Exchange of the two halves of every 16-lane row (row_ror:8).
__device__ __forceinline__ u32x4 swap_row_halves(const u32x4 &v) {
    return u32x4{(uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.x, 0x128, 0xF, 0xF, false),
                 (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.y, 0x128, 0xF, 0xF, false),
                 (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.z, 0x128, 0xF, 0xF, false),
                 (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.w, 0x128, 0xF, 0xF, false)};
}

// The MFMA input operands of a step: word column 2p is the loaded pair register as it is,
// word column 2p+1 the same register with its 16-lane row halves exchanged.  Either way
// the lanes of tokens 8..15 hold x of other tokens or columns: they only feed output
// columns 8..15 of the product, which no one reads.
template <int TT>
__device__ __forceinline__ void walk_tbatch(const TBatch<TT> &bt, const u32x4 (&xp)[kTStep / 2], uint8_t *tw, int lane,
                                            f32x4 (&acc)[TT]) {
    u32x4 xq[kTStep];
#pragma unroll
    for (int j = 0; j < kTStep / 2; ++j) {
        xq[2 * j] = xp[j];
        xq[2 * j + 1] = swap_row_halves(xp[j]);
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) walk_tile(bt.va[t], bt.vb[t], bt.ma[t], bt.mb[t], xq, tw, lane, acc[t]);
}

// Workgroup barrier for LDS traffic only: the weight loads in flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// End of a unit: the waves' partial sums go to LDS ([W][B][16*TT]), are added in wave
// order and stored.
template <int B, int EPI, int TT, int W>
__device__ __forceinline__ void finish_tile(f32x4 (&acc)[TT], float *red, const TileRows<TT> &tr,
                                            const SpmvSet &set, int wave, int lane) {
    constexpr int kR = kTRows * TT;  // partial sums per token and wave
    const int n = lane & 15, q = lane >> 4;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        if (n < B) *reinterpret_cast<f32x4 *>(red + (wave * B + n) * kR + kTRows * t + 4 * q) = acc[t];
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    lds_barrier();
    const int th = threadIdx.x;
    if constexpr (EPI == kEpiSwiGLU) {
        constexpr int kH = 8 * TT;  // outputs per token: gate/up row pairs of the unit
        if (th < kH * B) {
            const int j = th % kH, b = th / kH;
            const int gi = kTRows * (j >> 3) + (j & 7);  // gate row j sits in tile j/8, row j%8; up at row + 8
            float g = 0.f, u = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                g += red[(w * B + b) * kR + gi];
                u += red[(w * B + b) * kR + gi + 8];
            }
            if (tr.local + j < tr.rows) set.y[0][(int64_t)b * set.ldy[0] + tr.local + j] = f32_to_bf16_rne(silu_mul(g, u));
        }
    } else {
        if (th < kR * B) {
            const int i = th % kR, b = th / kR;
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) sum += red[(w * B + b) * kR + i];
            if (tr.local + i < tr.rows) set.y[tr.p][(int64_t)b * set.ldy[tr.p] + tr.local + i] = f32_to_bf16_rne(sum);
        }
    }
}

// W waves per workgroup share a unit of TT tiles (16*TT rows) at a time: the unit's
// steps of 4 words are dealt round-robin to the waves (wave w walks steps w, w + W,
// w + 2W, ...), one word of each tile per lane, all TT tiles of a step multiplied by the
// same x operand.  With the steps interleaved, the W waves read W consecutive 128-byte
// pieces of every row at about the same time -- runs of W*128 bytes per row instead of W
// pieces K/W columns apart -- which keeps the memory's row buffers busier (measured
// 4-13% faster at 8 tokens than contiguous quarters of K per wave).
template <int B, int EPI, int TT, int W>
__global__ __launch_bounds__(W * kWave, 4) void spmv_tile_kernel(const SpmvSet set, int KW,
                                                                 const uint16_t *__restrict__ x, int64_t ldx,
                                                                 int units) {
    extern __shared__ __attribute__((aligned(16))) uint8_t tlds[];
    uint8_t *dense = tlds;
    float *red0 = reinterpret_cast<float *>(tlds + (size_t)W * kTWaveBytes);
    float *red1 = red0 + W * B * kTRows * TT;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nwp = KW / W;  // words per wave and row; a multiple of kTStep
    const int steps = nwp / kTStep;
    const int my_units = (int)blockIdx.x < units ? (units - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
    const int total = my_units * steps;
    const uint32_t vo = (uint32_t)((lane >> 3) * KW * 32 + (lane & 7) * 16);
    const uint32_t mo = (uint32_t)((lane >> 3) * KW * 4 + ((lane & 7) >> 1) * 4);
    // x operand loads: lane l holds token (l & 7), k-block l >> 4 of word column 2p
    // (l & 15 < 8) or 2p+1 (l & 15 >= 8) -- all 64 lanes load, half the instructions of
    // one operand register per word column, and a token's two word columns are 128
    // contiguous bytes
    const int n = lane & 7;
    const uint32_t xo = n < B ? (uint32_t)(n * ldx * 2 + (lane >> 4) * 16 + ((lane >> 3) & 1) * 64) : kXOut;
    uint8_t *tw = dense + wave * kTWaveBytes;

    // Steps of this wave: (unit, step) for units blockIdx.x, + gridDim.x, ..., walked as
    // one flat sequence with the next step's loads in flight during the current one,
    // across unit boundaries too (two buffers used in turn, as in nm_spmv.hip).
    TBatch<TT> bA, bB;
    int tA = blockIdx.x, sA = 0, tB = tA, sB = 0;
    TileRows<TT> rA = tile_rows<EPI, TT>(set, min(tA, units - 1), KW), rB = rA;
    load_tbatch<B, TT>(bA, rA, wave * kTStep, KW, x, ldx, vo, mo, xo, total > 0);
    f32x4 acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    int buf = 0;
    int k = 0;
    for (; k + 1 < total; k += 2) {
        tB = tA;
        sB = sA + 1;
        if (sB == steps) {
            sB = 0;
            tB += gridDim.x;
            rB = tile_rows<EPI, TT>(set, min(tB, units - 1), KW);
        } else {
            rB = rA;
        }
        load_tbatch<B, TT>(bB, rB, (sB * W + wave) * kTStep, KW, x, ldx, vo, mo, xo, true);
        __builtin_amdgcn_sched_barrier(0);
        walk_tbatch<TT>(bA, bA.xp, tw, lane, acc);
        if (sA == steps - 1) {
            finish_tile<B, EPI, TT, W>(acc, buf ? red1 : red0, rA, set, wave, lane);
            buf ^= 1;
        }
        tA = tB;
        sA = sB + 1;
        if (sA == steps) {
            sA = 0;
            tA += gridDim.x;
            rA = tile_rows<EPI, TT>(set, min(tA, units - 1), KW);
        } else {
            rA = rB;
        }
        load_tbatch<B, TT>(bA, rA, (sA * W + wave) * kTStep, KW, x, ldx, vo, mo, xo, k + 2 < total);
        __builtin_amdgcn_sched_barrier(0);
        walk_tbatch<TT>(bB, bB.xp, tw, lane, acc);
        if (sB == steps - 1) {
            finish_tile<B, EPI, TT, W>(acc, buf ? red1 : red0, rB, set, wave, lane);
            buf ^= 1;
        }
    }
    if (k < total) {  // odd count: the last step is in A
        walk_tbatch<TT>(bA, bA.xp, tw, lane, acc);
        if (sA == steps - 1) finish_tile<B, EPI, TT, W>(acc, buf ? red1 : red0, rA, set, wave, lane);
    }
}

// One unit of the walk below.  Step s of the unit reads buffer A for even s and B for
// odd s; the last step loads the next unit's first step into A.  FIRST: the steps load
// their x operand with their weights, as in spmv_tile_kernel, and keep it in xc for the
// later units, which load weights only.
template <int B, int EPI, int TT, int W, int XC, bool FIRST>
__device__ __forceinline__ void xc_unit(TBatch<TT> &bA, TBatch<TT> &bB, u32x4 (&xc)[XC][kTStep / 2],
                                        const TileRows<TT> &r, const TileRows<TT> &rn, bool next_live, int KW,
                                        const uint16_t *x, int64_t ldx, uint32_t vo, uint32_t mo, uint32_t xo,
                                        int wave, uint8_t *tw, int lane, f32x4 (&acc)[TT]) {
#pragma unroll
    for (int s = 0; s < XC; s += 2) {
        load_tbatch<B, TT, FIRST>(bB, r, ((s + 1) * W + wave) * kTStep, KW, x, ldx, vo, mo, xo, true);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (FIRST) {
#pragma unroll
            for (int j = 0; j < kTStep / 2; ++j) xc[s][j] = bA.xp[j];
        }
        walk_tbatch<TT>(bA, xc[s], tw, lane, acc);
        if (s + 2 < XC)
            load_tbatch<B, TT, FIRST>(bA, r, ((s + 2) * W + wave) * kTStep, KW, x, ldx, vo, mo, xo, true);
        else
            load_tbatch<B, TT, false>(bA, rn, wave * kTStep, KW, x, ldx, vo, mo, xo, next_live);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (FIRST) {
#pragma unroll
            for (int j = 0; j < kTStep / 2; ++j) xc[s + 1][j] = bB.xp[j];
        }
        walk_tbatch<TT>(bB, xc[s + 1], tw, lane, acc);
    }
}

// The same walk where every wave has exactly XC steps per unit (K = 128 * W * XC
// columns, XC even): a wave's x columns are then the same in every unit, so it keeps
// them in registers (XC x 8 per lane) after its first unit, and the steps of its later
// units load weights only -- half the load instructions and L2 traffic of a one-tile
// step.  The first unit loads x step by step with the weights, so a workgroup with a
// single unit waits no longer for its first step than spmv_tile_kernel does.
template <int B, int EPI, int TT, int W, int XC>
__global__ __launch_bounds__(W * kWave, 4) void spmv_tile_xc_kernel(const SpmvSet set, int KW,
                                                                    const uint16_t *__restrict__ x, int64_t ldx,
                                                                    int units) {
    static_assert(XC % 2 == 0, "steps per unit alternate between the two buffers");
    extern __shared__ __attribute__((aligned(16))) uint8_t tlds[];
    uint8_t *dense = tlds;
    float *red0 = reinterpret_cast<float *>(tlds + (size_t)W * kTWaveBytes);
    float *red1 = red0 + W * B * kTRows * TT;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t vo = (uint32_t)((lane >> 3) * KW * 32 + (lane & 7) * 16);
    const uint32_t mo = (uint32_t)((lane >> 3) * KW * 4 + ((lane & 7) >> 1) * 4);
    const int n = lane & 7;  // x operand lanes as in spmv_tile_kernel
    const uint32_t xo = n < B ? (uint32_t)(n * ldx * 2 + (lane >> 4) * 16 + ((lane >> 3) & 1) * 64) : kXOut;
    uint8_t *tw = dense + wave * kTWaveBytes;

    // the wave's x operand of each of its XC steps (word column (s * W + wave) * 4)
    u32x4 xc[XC][kTStep / 2];
    TBatch<TT> bA, bB;
    f32x4 acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the grid never exceeds the units, so every workgroup has at least one
    int u = blockIdx.x;
    TileRows<TT> r = tile_rows<EPI, TT>(set, u, KW);
    load_tbatch<B, TT, true>(bA, r, wave * kTStep, KW, x, ldx, vo, mo, xo, true);
    {
        const int un = u + gridDim.x;
        const TileRows<TT> rn = tile_rows<EPI, TT>(set, min(un, units - 1), KW);
        xc_unit<B, EPI, TT, W, XC, true>(bA, bB, xc, r, rn, un < units, KW, x, ldx, vo, mo, xo, wave, tw, lane, acc);
        finish_tile<B, EPI, TT, W>(acc, red0, r, set, wave, lane);
        r = rn;
        u = un;
    }
    int buf = 1;
    for (; u < units; u += gridDim.x) {
        const int un = u + gridDim.x;
        const TileRows<TT> rn = tile_rows<EPI, TT>(set, min(un, units - 1), KW);
        xc_unit<B, EPI, TT, W, XC, false>(bA, bB, xc, r, rn, un < units, KW, x, ldx, vo, mo, xo, wave, tw, lane, acc);
        finish_tile<B, EPI, TT, W>(acc, buf ? red1 : red0, r, set, wave, lane);
        buf ^= 1;
        r = rn;
    }
}

// Raise the dynamic-LDS limit of one kernel instance once per device.
template <int B, int TT, int W>
hipError_t allow_tile_lds(const void *kernel, std::atomic<uint64_t> &done) {
    constexpr size_t bytes = tile_lds_bytes<B, TT, W>();
    if (bytes <= 64 * 1024) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = 1ull << (dev & 63);
    if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

// Steps per wave and unit for which the x operand is held in registers.
constexpr int kTileXC = 4;

template <int B, int EPI, int TT, int W>
hipError_t launch_tbw(const MvPlan &p, const SpmvSet &set, int64_t K, const uint16_t *x, int64_t ldx,
                      hipStream_t st) {
    SpmvSet padded = set;
    for (int q = set.P + 1; q <= kMaxMats; ++q) padded.row0[q] = set.row0[set.P];
    const int KW = (int)(K / 32);
    if (p.xreg) {
        if (p.xreg != kTileXC || KW != W * kTStep * kTileXC) return hipErrorInvalidValue;
        static std::atomic<uint64_t> done{0};
        const void *kern = (const void *)spmv_tile_xc_kernel<B, EPI, TT, W, kTileXC>;
        hipError_t e = allow_tile_lds<B, TT, W>(kern, done);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((spmv_tile_xc_kernel<B, EPI, TT, W, kTileXC>), dim3((unsigned)p.grid_x), dim3(W * kWave),
                           (tile_lds_bytes<B, TT, W>()), st, padded, KW, x, ldx, p.tiles);
        return hipGetLastError();
    }
    static std::atomic<uint64_t> done{0};
    hipError_t e = allow_tile_lds<B, TT, W>((const void *)spmv_tile_kernel<B, EPI, TT, W>, done);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((spmv_tile_kernel<B, EPI, TT, W>), dim3((unsigned)p.grid_x), dim3(W * kWave),
                       (tile_lds_bytes<B, TT, W>()), st, padded, KW, x, ldx, p.tiles);
    return hipGetLastError();
}

template <int B, int EPI>
hipError_t launch_tb(const MvPlan &p, const SpmvSet &set, int64_t K, const uint16_t *x, int64_t ldx,
                     hipStream_t st) {
    const int tt = p.unroll, w = p.threads / kWave;
    if (tt == 2 && w == 16) return launch_tbw<B, EPI, 2, 16>(p, set, K, x, ldx, st);
    if (tt == 2 && w == 8) return launch_tbw<B, EPI, 2, 8>(p, set, K, x, ldx, st);
    if (tt == 1 && w == 16) return launch_tbw<B, EPI, 1, 16>(p, set, K, x, ldx, st);
    if (tt == 1 && w == 8) return launch_tbw<B, EPI, 1, 8>(p, set, K, x, ldx, st);
    return hipErrorInvalidValue;
}

template <int EPI>
hipError_t launch_te(const MvPlan &p, const SpmvSet &set, int64_t K, const uint16_t *x, int64_t ldx, int B,
                     hipStream_t st) {
    switch (B) {
    case 3: return launch_tb<3, EPI>(p, set, K, x, ldx, st);
    case 4: return launch_tb<4, EPI>(p, set, K, x, ldx, st);
    case 5: return launch_tb<5, EPI>(p, set, K, x, ldx, st);
    case 6: return launch_tb<6, EPI>(p, set, K, x, ldx, st);
    case 7: return launch_tb<7, EPI>(p, set, K, x, ldx, st);
    case 8: return launch_tb<8, EPI>(p, set, K, x, ldx, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool spmv_tile_ok(const SpmvSet &set, int64_t K, int64_t ldx, int B, int fmt, int epi) {
    if (fmt != kMetaBitmask || B < kTileLowB || B > 8) return false;
    if (K % (32 * 8 * kTStep) != 0) return false;  // every wave of an 8-wave workgroup gets whole steps
    // 32-bit buffer offsets: 8 rows of values, and the x rows of all tokens
    if ((int64_t)8 * K > ((int64_t)1 << 30) || (int64_t)(B - 1) * ldx * 2 + K * 2 > ((int64_t)1 << 30)) return false;
    if (epi == kEpiSwiGLU) return set.P == 2 && set.row0[2] == 2 * set.row0[1];
    for (int p = 1; p < set.P; ++p)
        if (set.row0[p] % kTRows) return false;  // tiles must not straddle two matrices
    return true;
}

MvPlan plan_spmv_tile(const SpmvSet &set, int64_t K, int B, const DeviceInfo &dev, int epi) {
    MvPlan p;
    p.tile = 1;
    const int64_t R = set.row0[set.P];
    const int64_t cu = dev.num_cu > 0 ? dev.num_cu : 256;
    const int64_t tiles = epi == kEpiSwiGLU ? (R / 2 + 7) / 8 : (R + kTRows - 1) / kTRows;
    // Two 8-wave workgroups per CU (LDS and register budget), or one 16-wave workgroup
    // per CU -- as many waves in flight -- where K gives every one of 16 waves at least
    // four steps per tile and
    //   * there are fewer tiles than 8-wave workgroups, or
    //   * every wave of 16 then has exactly kTileXC steps (x stays in registers after a
    //     workgroup's first unit) and either 7 or 8 tokens make x a large share of the
    //     loads (28672 x 8192, 8 tokens: 56.7 -> 52.1 us; 12288 x 8192, 7 tokens: 25.0 ->
    //     24.5 us; 5 and 6 tokens on 3 or more tiles per CU: 2-6% slower, so not there) or
    //     there are at most two tiles per CU (8192 x 8192: 18.7 -> 17.7 us at 8 tokens,
    //     17.8 -> 17.3 at 5), or
    //   * K is long (8 or more steps per wave of 16): the x operand, re-read every step,
    //     is then shared by two tiles from as few as 2 tiles per CU on (8 tokens,
    //     8192 x 28672: 60.2 -> 53.7 us).
    const int64_t s16 = K % (32 * 16 * kTStep) == 0 ? K / (32 * 16 * kTStep) : 0;  // steps per wave of 16
    const bool w16 = s16 >= 4 && (tiles < 2 * cu || (s16 == kTileXC && (B >= 7 || tiles <= 2 * cu)) || s16 >= 8);
    const int w = w16 ? 16 : 8;
    const int64_t slots = cu * (16 / w);  // resident workgroups
    // Two tiles per step (one x operand for 32 rows, half the x loads per weight byte)
    // when that leaves the CUs as evenly loaded as one tile per step does: the units of
    // work per CU are whole, and a CU's last unit is the launch's tail.
    bool two = (tiles + 1) / 2 >= slots;
    if (epi != kEpiSwiGLU)
        for (int q = 1; q < set.P; ++q)
            if (set.row0[q] % (2 * kTRows)) two = false;  // units must not straddle two matrices
    if (two) {
        const int64_t u1 = tiles, u2 = (tiles + 1) / 2;
        // ceil(u / cu) / (u / cu): compare ceil(u2/cu) * u1 with ceil(u1/cu) * u2
        if ((u2 + cu - 1) / cu * u1 > (u1 + cu - 1) / cu * u2) two = false;
        // with x kept in registers, a workgroup's later units reuse its x operand: one
        // tile per step and two units per workgroup beat two tiles and a single unit
        // (8192 x 8192, 16 waves, 8 tokens: 17.8 vs 18.4 us)
        if (K / 32 == (int64_t)w * kTStep * kTileXC && u2 <= slots) two = false;
    }
    const int tt = two ? 2 : 1;
    const int64_t units = (tiles + tt - 1) / tt;
    int64_t gx = slots;
    if (gx > units) gx = units;
    p.grid_x = (int)(gx < 1 ? 1 : gx);
    p.tiles = (int)units;
    p.unroll = tt;
    p.threads = w * kWave;
    p.xreg = K / 32 == (int64_t)w * kTStep * kTileXC ? kTileXC : 0;
    p.splits = 1;
    p.ws_bytes = 0;
    return p;
}

hipError_t launch_spmv_tile(const MvPlan &p, const SpmvSet &set, int64_t K, const uint16_t *x, int64_t ldx, int B,
                            int epi, hipStream_t st) {
    if (epi == kEpiSwiGLU) return launch_te<kEpiSwiGLU>(p, set, K, x, ldx, B, st);
    return launch_te<kEpiNone>(p, set, K, x, ldx, B, st);
}

}  // namespace nmk
