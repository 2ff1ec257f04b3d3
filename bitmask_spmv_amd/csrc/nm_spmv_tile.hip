// nm_spmv_tile.hip -- N:M sparse matrix times a small batch of input vectors (5..8 tokens)
// with the products on the matrix cores of gfx950.
//
// What it computes: the same product as nm_spmv.hip, over the same packed operands --
// one 32-bit mask word per 32 columns whose set bits pair, in increasing column order,
// with the stored values ("SparseDecoding: Decoding-Aware Pruning ..." (ai.info summary),
// Methodology Steps 2-3; "SparseDecoding:解码感知的准确高效大模型剪枝框架"
// (paper.rainbus.top), 方法步骤详情 第四步) -- for B = 5..8 input vectors.
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
//   * a workgroup (8 waves) owns a tile of 16 rows at a time; wave w walks words
//     [w*KW/8, (w+1)*KW/8) of those rows in steps of 4 words, one word per lane;
//   * tile rows 0-7 and 8-15 are 8 consecutive rows of one matrix each (plain launch:
//     the same matrix; gated MLP: gate rows i..i+7, then up rows i..i+7);
//   * a step loads 128 bytes of values per row (two 16-byte loads per lane, rows 0-7
//     then rows 8-15, 8 lanes per row, contiguous), the lane's mask word of both row
//     halves, and the step's 4 x 32 columns of x straight into the MFMA operand
//     registers (x is re-read by every tile: an L2 hit); a swap of 16-byte halves between
//     lane pairs gives each lane the 16 values of its word, as in nm_spmv.hip;
//   * the lane zeroes its word's 32 columns of the wave's dense tile and writes its 16
//     kept values at their columns; four MFMAs then add the step into the wave's 16xB
//     accumulator (lane l: rows 4*(l/16)..+3 of token l%16);
//   * at the end of a tile the 8 waves' partial sums meet in LDS and are added in wave
//     order (deterministic), then rounded once to bf16 -- for the gated MLP combined
//     first as silu(gate) * up.
// Every load goes through a raw buffer descriptor whose base carries the step's column
// offset and whose size ends at the last valid row, so rows past the matrix, token lanes
// past B and the one batch issued past the end of the work read zeros without touching
// memory, and every wave issues the same loads in the same order.
#include "nm_device.h"
#include "nm_kernels.h"
#include "nm_spmv_common.h"

namespace nmk {
namespace {

constexpr int kTWaves = 8;
constexpr int kTThreads = kTWaves * kWave;
constexpr int kTRows = 16;                        // rows per tile (the MFMA's M)
constexpr int kTStep = 4;                         // words per row and step
constexpr int kTRowBytes = 16 + kTStep * 64;      // tile row: 16-byte lead pad + 4 x 32 bf16
constexpr int kTWaveBytes = kTRows * kTRowBytes + 16;  // one wave's dense tile + a 16-byte tail pad
constexpr uint32_t kXOut = 0x40000000u;           // x offset of token lanes >= B: past the buffer

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// One step's loads (64 words: 4 words of each of the 16 rows).
struct TBatch {
    u32x4 va, vb;      // 16-byte value chunk (lane & 7) of row (lane >> 3), of row 8 + (lane >> 3)
    uint32_t ma, mb;   // mask word ((lane & 7) >> 1) of the same two rows
    u32x4 xq[kTStep];  // MFMA input operand of the step's four word columns
};

// Where a tile's rows live, and where its outputs go.
struct TileRows {
    const uint8_t *m[2];  // masks of the first row of each half
    const uint8_t *v[2];  // values of the first row of each half
    int valid[2];         // rows of each half inside the matrix (0..8)
    int p;                // output matrix
    int local;            // first output row of the tile within matrix p
    int rows;             // rows of matrix p (plain launch) / of the gate matrix (gated MLP)
};

template <int EPI>
__device__ __forceinline__ TileRows tile_rows(const SpmvSet &set, int tile, int KW) {
    TileRows t;
    if constexpr (EPI == kEpiSwiGLU) {
        const int i0 = tile * 8;
        const int n = min(max(set.row0[1] - i0, 0), 8);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            t.m[h] = static_cast<const uint8_t *>(set.meta[h]) + (int64_t)i0 * KW * 4;
            t.v[h] = reinterpret_cast<const uint8_t *>(set.values[h]) + (int64_t)i0 * KW * 32;
            t.valid[h] = n;
        }
        t.p = 0;
        t.local = i0;
        t.rows = set.row0[1];
    } else {
        const int tb = tile * kTRows;
        const int p = owner(set, tb);  // a tile never straddles two matrices
        const int lb = tb - set.row0[p];
        const int rp = set.row0[p + 1] - set.row0[p];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            t.m[h] = static_cast<const uint8_t *>(set.meta[p]) + (int64_t)(lb + 8 * h) * KW * 4;
            t.v[h] = reinterpret_cast<const uint8_t *>(set.values[p]) + (int64_t)(lb + 8 * h) * KW * 32;
            t.valid[h] = min(max(rp - lb - 8 * h, 0), 8);
        }
        t.p = p;
        t.local = lb;
        t.rows = rp;
    }
    return t;
}

// Loads of one step at word column cw (live = false: the same loads with empty ranges).
template <int B>
__device__ __forceinline__ void load_tbatch(TBatch &bt, const TileRows &tr, int cw, int KW, const uint16_t *x,
                                            int64_t ldx, uint32_t vo, uint32_t mo, uint32_t xo, bool live) {
    const int64_t vrow = (int64_t)KW * 32, mrow = (int64_t)KW * 4;
    const int64_t vn0 = live ? tr.valid[0] * vrow - (int64_t)cw * 32 : 0;
    const int64_t vn1 = live ? tr.valid[1] * vrow - (int64_t)cw * 32 : 0;
    const int64_t mn0 = live ? tr.valid[0] * mrow - (int64_t)cw * 4 : 0;
    const int64_t mn1 = live ? tr.valid[1] * mrow - (int64_t)cw * 4 : 0;
    const int64_t xn = live ? (int64_t)(B - 1) * ldx * 2 + (int64_t)(KW - cw) * 64 : 0;
    const __amdgpu_buffer_rsrc_t rv0 = make_rsrc(tr.v[0] + (int64_t)cw * 32, vn0 > 0 ? vn0 : 0);
    const __amdgpu_buffer_rsrc_t rv1 = make_rsrc(tr.v[1] + (int64_t)cw * 32, vn1 > 0 ? vn1 : 0);
    const __amdgpu_buffer_rsrc_t rm0 = make_rsrc(tr.m[0] + (int64_t)cw * 4, mn0 > 0 ? mn0 : 0);
    const __amdgpu_buffer_rsrc_t rm1 = make_rsrc(tr.m[1] + (int64_t)cw * 4, mn1 > 0 ? mn1 : 0);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (int64_t)cw * 32, xn);
    bt.va = __builtin_amdgcn_raw_buffer_load_b128(rv0, vo, 0, kLoadNT);
    bt.vb = __builtin_amdgcn_raw_buffer_load_b128(rv1, vo, 0, kLoadNT);
    bt.ma = __builtin_amdgcn_raw_buffer_load_b32(rm0, mo, 0, kLoadNT);
    bt.mb = __builtin_amdgcn_raw_buffer_load_b32(rm1, mo, 0, kLoadNT);
#pragma unroll
    for (int j = 0; j < kTStep; ++j) bt.xq[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo + j * 64u, 0, 0);
}

// Swap one dword with the neighbouring lane of the pair (lane ^ 1).
__device__ __forceinline__ uint32_t tpair_swap(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // quad_perm(1,0,3,2)
}

// One step: expand the lane's word into the wave's dense tile, then four MFMAs.
//
// Lane l's word: row (l & 1) * 8 + (l >> 3) of the tile, word column (l & 7) >> 1.  Its
// 32 columns are zeroed and its 16 kept values written at their columns.  Even lanes
// walk the word from its lowest set bit up, odd lanes from its highest set bit down (the
// lowest set bit of the bit-reversed mask, the values taken in reverse order): at each
// of the 16 steps the lanes then write near opposite ends of their words, which spreads
// the writes of lanes whose words start on the same LDS bank.  A word whose mask runs out
// of set bits (only rows past the matrix, whose loads read zero) writes one column before
// the word (even lanes) or one after it (odd lanes): the row's lead pad, the neighbouring
// word of the same row, the next row's lead pad or the tile's tail pad -- never another
// row's data or another wave's tile.  The zeroing writes of lanes with rows 8..15 take
// the word's 16-byte chunks in the order 2, 3, 0, 1, so the 16 lanes of each group of a
// 16-byte write cover distinct banks.  The wave's LDS operations execute in issue order,
// so the expansion is complete before the operand reads that follow it.
__device__ __forceinline__ void walk_tbatch(const TBatch &bt, uint8_t *tw, int lane, f32x4 &acc) {
    const bool odd = lane & 1;
    const uint32_t s_x = odd ? bt.va.x : bt.vb.x, s_y = odd ? bt.va.y : bt.vb.y;
    const uint32_t s_z = odd ? bt.va.z : bt.vb.z, s_w = odd ? bt.va.w : bt.vb.w;
    const uint32_t r_x = tpair_swap(s_x), r_y = tpair_swap(s_y), r_z = tpair_swap(s_z), r_w = tpair_swap(s_w);
    // the word's 16 values in walk order: even lanes ascending, odd lanes descending
    // (dword d of the odd lane = the two values of dword 7 - d, halves swapped)
    const uint32_t od[8] = {bt.vb.w, bt.vb.z, bt.vb.y, bt.vb.x, r_w, r_z, r_y, r_x};
    const uint32_t ev[8] = {bt.va.x, bt.va.y, bt.va.z, bt.va.w, r_x, r_y, r_z, r_w};
    uint32_t v[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) v[d] = odd ? __builtin_amdgcn_alignbit(od[d], od[d], 16) : ev[d];
    uint32_t m = odd ? __builtin_bitreverse32(bt.mb) : bt.ma;
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
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, bt.xq[j]),
                                                      acc, 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
}

// Workgroup barrier for LDS traffic only: the weight loads in flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// End of a tile: the waves' partial sums go to LDS, are added in wave order and stored.
template <int B, int EPI>
__device__ __forceinline__ void finish_tile(f32x4 &acc, float (*red)[B][kTRows], const TileRows &tr,
                                            const SpmvSet &set, int wave, int lane) {
    const int n = lane & 15, q = lane >> 4;
    if (n < B) *reinterpret_cast<f32x4 *>(&red[wave][n][4 * q]) = acc;
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    lds_barrier();
    const int t = threadIdx.x;
    if constexpr (EPI == kEpiSwiGLU) {
        if (t < 8 * B) {
            const int j = t & 7, b = t >> 3;
            float g = 0.f, u = 0.f;
#pragma unroll
            for (int w = 0; w < kTWaves; ++w) {
                g += red[w][b][j];
                u += red[w][b][8 + j];
            }
            if (tr.local + j < tr.rows) set.y[0][(int64_t)b * set.ldy[0] + tr.local + j] = f32_to_bf16_rne(silu_mul(g, u));
        }
    } else {
        if (t < kTRows * B) {
            const int i = t & 15, b = t >> 4;
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < kTWaves; ++w) s += red[w][b][i];
            if (tr.local + i < tr.rows) set.y[tr.p][(int64_t)b * set.ldy[tr.p] + tr.local + i] = f32_to_bf16_rne(s);
        }
    }
}

template <int B, int EPI>
__global__ __launch_bounds__(kTThreads, 4) void spmv_tile_kernel(const SpmvSet set, int KW,
                                                                 const uint16_t *__restrict__ x, int64_t ldx,
                                                                 int tiles) {
    __shared__ __attribute__((aligned(16))) uint8_t dense[kTWaves * kTWaveBytes];
    __shared__ __attribute__((aligned(16))) float red[2][kTWaves][B][kTRows];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nwp = KW / kTWaves;  // words per wave and row; a multiple of kTStep
    const int steps = nwp / kTStep;
    const int wa = wave * nwp;
    const int my_tiles = (int)blockIdx.x < tiles ? (tiles - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
    const int total = my_tiles * steps;
    const uint32_t vo = (uint32_t)((lane >> 3) * KW * 32 + (lane & 7) * 16);
    const uint32_t mo = (uint32_t)((lane >> 3) * KW * 4 + ((lane & 7) >> 1) * 4);
    const int n = lane & 15;
    const uint32_t xo = n < B ? (uint32_t)(n * ldx * 2 + (lane >> 4) * 16) : kXOut;
    uint8_t *tw = dense + wave * kTWaveBytes;

    // Steps of this wave: (tile, step) for tiles blockIdx.x, + gridDim.x, ..., walked as
    // one flat sequence with the next step's loads in flight during the current one,
    // across tile boundaries too (two buffers used in turn, as in nm_spmv.hip).
    TBatch bA, bB;
    int tA = blockIdx.x, sA = 0, tB = tA, sB = 0;
    TileRows rA = tile_rows<EPI>(set, min(tA, tiles - 1), KW), rB = rA;
    load_tbatch<B>(bA, rA, wa, KW, x, ldx, vo, mo, xo, total > 0);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int buf = 0;
    int k = 0;
    for (; k + 1 < total; k += 2) {
        tB = tA;
        sB = sA + 1;
        if (sB == steps) {
            sB = 0;
            tB += gridDim.x;
            rB = tile_rows<EPI>(set, min(tB, tiles - 1), KW);
        } else {
            rB = rA;
        }
        load_tbatch<B>(bB, rB, wa + kTStep * sB, KW, x, ldx, vo, mo, xo, true);
        __builtin_amdgcn_sched_barrier(0);
        walk_tbatch(bA, tw, lane, acc);
        if (sA == steps - 1) {
            finish_tile<B, EPI>(acc, red[buf], rA, set, wave, lane);
            buf ^= 1;
        }
        tA = tB;
        sA = sB + 1;
        if (sA == steps) {
            sA = 0;
            tA += gridDim.x;
            rA = tile_rows<EPI>(set, min(tA, tiles - 1), KW);
        } else {
            rA = rB;
        }
        load_tbatch<B>(bA, rA, wa + kTStep * sA, KW, x, ldx, vo, mo, xo, k + 2 < total);
        __builtin_amdgcn_sched_barrier(0);
        walk_tbatch(bB, tw, lane, acc);
        if (sB == steps - 1) {
            finish_tile<B, EPI>(acc, red[buf], rB, set, wave, lane);
            buf ^= 1;
        }
    }
    if (k < total) {  // odd count: the last step is in A
        walk_tbatch(bA, tw, lane, acc);
        if (sA == steps - 1) finish_tile<B, EPI>(acc, red[buf], rA, set, wave, lane);
    }
}

template <int B, int EPI>
hipError_t launch_tb(const MvPlan &p, const SpmvSet &set, int64_t K, const uint16_t *x, int64_t ldx,
                     hipStream_t st) {
    SpmvSet padded = set;
    for (int q = set.P + 1; q <= kMaxMats; ++q) padded.row0[q] = set.row0[set.P];
    hipLaunchKernelGGL((spmv_tile_kernel<B, EPI>), dim3((unsigned)p.grid_x), dim3(kTThreads), 0, st, padded,
                       (int)(K / 32), x, ldx, p.tiles);
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_te(const MvPlan &p, const SpmvSet &set, int64_t K, const uint16_t *x, int64_t ldx, int B,
                     hipStream_t st) {
    switch (B) {
    case 5: return launch_tb<5, EPI>(p, set, K, x, ldx, st);
    case 6: return launch_tb<6, EPI>(p, set, K, x, ldx, st);
    case 7: return launch_tb<7, EPI>(p, set, K, x, ldx, st);
    case 8: return launch_tb<8, EPI>(p, set, K, x, ldx, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool spmv_tile_ok(const SpmvSet &set, int64_t K, int64_t ldx, int B, int fmt, int epi) {
    if (fmt != kMetaBitmask || B < kTileMinB || B > 8) return false;
    if (K % (32 * kTWaves * kTStep) != 0) return false;  // every wave gets whole steps
    // 32-bit buffer offsets: 8 rows of values, and the x rows of all tokens
    if ((int64_t)8 * K > ((int64_t)1 << 30) || (int64_t)(B - 1) * ldx * 2 + K * 2 > ((int64_t)1 << 30)) return false;
    if (epi == kEpiSwiGLU) return set.P == 2 && set.row0[2] == 2 * set.row0[1];
    for (int p = 1; p < set.P; ++p)
        if (set.row0[p] % kTRows) return false;  // tiles must not straddle two matrices
    return true;
}

MvPlan plan_spmv_tile(int64_t R, int B, const DeviceInfo &dev, int epi) {
    (void)B;
    MvPlan p;
    p.tile = 1;
    p.threads = kTThreads;
    const int64_t tiles = epi == kEpiSwiGLU ? (R / 2 + 7) / 8 : (R + kTRows - 1) / kTRows;
    const int64_t cu = dev.num_cu > 0 ? dev.num_cu : 256;
    int64_t gx = cu * 2;  // two 8-wave workgroups per CU (LDS and register budget)
    if (gx > tiles) gx = tiles;
    p.grid_x = (int)(gx < 1 ? 1 : gx);
    p.tiles = (int)tiles;
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
