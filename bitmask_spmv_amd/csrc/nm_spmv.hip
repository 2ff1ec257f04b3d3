// nm_spmv.hip -- batch-one / small-batch N:M sparse matrix-vector product on gfx950.
//
// What it computes (pages cited by title and section):
//   "SparseDecoding: Decoding-Aware Pruning ..." (ai.info summary), Methodology Steps 2-3:
//     each 32-bit mask word marks the kept columns of 32 consecutive inputs; its set
//     bits pair one-to-one, in increasing column order, with the stored values; at 50%
//     N:M with M <= 32 every aligned word has exactly 16 set bits, so the walk over a
//     word is a fixed 16-step loop of "lowest set bit -> column, clear it".
//   "SparseDecoding:解码感知的准确高效大模型剪枝框架" (paper.rainbus.top), 方法步骤详情
//     第四步: the input vector is the reused operand and weights/masks are streamed;
//     rows may be split with a reduction of the pieces.  核心方法 (核心创新二): the
//     bitmask costs 2 bits per kept weight against 8 for a uint8 offset and 32 for an
//     int32 column index; both index formats run on the same kernel skeleton (the
//     metadata format is a template parameter) so the trade-off can be measured.
//
// gfx950 design (what differs from the pages' A100/Triton kernel):
//   * x lives in LDS for the whole workgroup: each 32-column block of x occupies 17
//     dwords (16 data + 1 pad), so lanes that walk consecutive words land on different
//     banks even when their bit positions agree.
//   * word-per-lane mapping on the canonical row-major layout: each lane of a wave takes
//     one word of a 64-word strip of the row, so one wave iteration loads 256 contiguous
//     bytes of masks and 2 KiB of contiguous values (two 16-byte loads per lane), all
//     non-temporal; the next strip's loads go out before the current strip is walked.
//   * 16 steps per word = 8 pairs; each pair gathers two bf16 inputs from LDS into one
//     dword and feeds v_dot2_f32_bf16 with the matching packed value pair.
//   * each wave owns whole rows (or row slices); the row total is a wave64 reduction.
//     Slices of a row (when splits > 1) go to fp32 workspace and are added in slice
//     order by a second kernel (deterministic, no atomics).  One-token rows of 7 or more
//     strips may instead be walked by two waves of a workgroup, half the strips each,
//     the two totals added in LDS in half order.
//   * one kernel serves every 50% pattern (2:4 ... 16:32): the M of the pattern never
//     enters the traversal.  Several matrices that share x run in one launch (SpmvSet).
#include <atomic>
#include <mutex>

#include <type_traits>

#include "nm_device.h"
#include "nm_kernels.h"
#include "nm_spmv_common.h"

namespace nmk {
namespace {

constexpr int kThreads = 512;     // default workgroup: 8 waves (256 for matrices with few rows)

// 1024-thread workgroups (16 waves, at most 64 VGPRs so two fit per CU) for the launches
// whose x slice leaves room for only two workgroups per CU: the bitmask kernel at B = 3
// and 4 fits that register budget without spilling (measured 4-9% faster on the 70B
// shapes at B = 4); B >= 5 and the index formats would spill.
constexpr bool wide_ok(int fmt, int B) { return fmt == kMetaBitmask && B <= 4; }
constexpr size_t kLdsCap = 80 * 1024;     // keeps two workgroups resident per CU
constexpr size_t kLdsPerCu = 160 * 1024;  // gfx950 LDS per compute unit

// Metadata bytes per 32-column word (16 kept weights) of each format.
constexpr int meta_bytes(int fmt) { return fmt == kMetaBitmask ? 4 : (fmt == kMetaU8 ? 16 : 64); }

// One wave-iteration batch: a 64-word strip of one row slice.
//
// Bitmask and uint8 offsets -- one word per lane.  Each 16-byte value load is contiguous
// across the wave (lane l reads chunk l of the strip's first KiB, then chunk l of its
// second KiB), which halves the cache lines each load instruction touches compared with
// one lane reading a whole 32-byte word; a quad-permute then swaps halves between lane
// pairs so that lane 2i ends up with word i and lane 2i+1 with word 32+i.  Each lane
// loads its own word's metadata (4 or 16 bytes; the 16-byte offset loads of the wave
// cover one contiguous KiB).
//
// int32 indices -- one quarter-word per lane and load.  A word's 64 bytes of indices
// would take four 16-byte loads per lane at a 64-byte lane stride; instead load q
// (q = 0..3) gives lane l the indices of kept weights 4(l%4)..4(l%4)+3 of word
// 16q + l/4 (contiguous 1 KiB across the wave) and the matching 8 bytes of values
// (contiguous 512 bytes).  Every lane then walks four entries of four words of the
// same row; the row total does not care which lane holds which product.
template <int FMT>
struct Batch {
    u32x4 va, vb;                          // values: two 16-byte chunks, or four 8-byte pieces (int32)
    u32x4 meta[FMT == kMetaI32 ? 4 : 1];   // mask (.x) / 16 offsets / four quarter-words of indices
    int lw;  // (first) word of this lane within the slice; >= the slice length marks padding
};

// Loads one batch through raw buffer descriptors covering the row slice's `words`
// words (0 = nothing to load: the loads still issue and return zeros, as do lanes
// past the end of the slice).
template <int FMT>
__device__ __forceinline__ void load_batch(Batch<FMT> &bt, const uint8_t *mrow, const u32x4 *vrow, int words,
                                           int base, int lane) {
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(mrow, (int64_t)words * meta_bytes(FMT));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vrow, (int64_t)words * 32);
    if constexpr (FMT == kMetaI32) {
        u32x2 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bt.meta[q] = __builtin_amdgcn_raw_buffer_load_b128(rm, base * 64 + 1024 * q + 16 * lane, 0, kLoadNT);
            v[q] = __builtin_amdgcn_raw_buffer_load_b64(rv, base * 32 + 512 * q + 8 * lane, 0, kLoadNT);
        }
        bt.va = u32x4{v[0].x, v[0].y, v[1].x, v[1].y};
        bt.vb = u32x4{v[2].x, v[2].y, v[3].x, v[3].y};
        bt.lw = base + (lane >> 2);
    } else {
        const int w = base + ((lane & 1) ? 32 + (lane >> 1) : (lane >> 1));
        if constexpr (FMT == kMetaBitmask)
            bt.meta[0].x = __builtin_amdgcn_raw_buffer_load_b32(rm, w * 4, 0, kLoadNT);
        else
            bt.meta[0] = __builtin_amdgcn_raw_buffer_load_b128(rm, w * 16, 0, kLoadNT);
        bt.va = __builtin_amdgcn_raw_buffer_load_b128(rv, base * 32 + lane * 16, 0, kLoadNT);
        bt.vb = __builtin_amdgcn_raw_buffer_load_b128(rv, base * 32 + 1024 + lane * 16, 0, kLoadNT);
        bt.lw = w;
    }
}

// Swap one dword with the neighbouring lane of the pair (lane ^ 1).  Every lane has a
// source lane, so the "old" operand is never read; passing v itself saves the compiler a
// register set to zero where v is not needed afterwards.
__device__ __forceinline__ uint32_t pair_swap(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false);  // quad_perm(1,0,3,2)
}

// Walk of one batch: 8 pairs of kept weights per lane.
//
// Columns within the word: bitmask -- the fixed 16-step walk, lowest set bit gives the
// column and is then cleared; uint8 -- byte t of the word's offsets; int32 -- at 50% N:M
// an index of word w always lies in [32w, 32w + 32), so its low five bits are the column
// within the word.  The index formats are masked to five bits so that no metadata value
// can address outside the word's block of x.
//
// A padding lane (past the slice) holds zero values and walks fixed columns of block 0
// (bitmask: the low 16 columns; index formats: zero metadata, column 0), so every LDS
// address stays inside the staged x.  A bitmask word without exactly 16 set bits (outside
// the input contract) walks the low 16 columns of its own block instead, so each of the
// 16 bit scans finds a set bit.
//
// One token (bitmask and uint8 offsets; blocked x): no value exchange between the lanes
// of a pair.  Lane 2i holds values 0..7 of words i and 32+i of the strip (the first
// halves of its two 16-byte chunks), lane 2i+1 values 8..15 of the same two words, and
// each walks its eight values of both words: even lanes from the lowest kept column up,
// odd lanes from the highest down (the lowest set bits of the bit-reversed mask word; for
// uint8 the offset bytes in reverse order).  Only the partner's metadata crosses lanes
// (one or two DPP moves), and each lane runs two independent chains of eight steps.  The
// bitmask and uint8 walks visit the same kept weights in the same order on the same
// lane, so their fp32 sums agree bit for bit.
//
// Two or more tokens (panel x): the exchange of value halves below gives every lane one
// whole word, lane 2i word i and lane 2i+1 word 32+i, and the panel layout gives each
// lane's block LDS banks of its own (measured against the walk without exchange on
// blocked x at two tokens: 1-6% faster on the Llama-3.1-8B and -3.3-70B shapes).
template <int FMT, int B>
__device__ __forceinline__ void walk_batch(const Batch<FMT> &bt, const uint32_t *xs, int nws, float (&acc)[B]) {
    constexpr int kBlk = XLayout<B>::kBlk;
    constexpr bool kPanel = B >= 2;  // x in the panel layout (else blocked)
    if constexpr (FMT == kMetaI32) {
        const uint32_t v[8] = {bt.va.x, bt.va.y, bt.va.z, bt.va.w, bt.vb.x, bt.vb.y, bt.vb.z, bt.vb.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int w = bt.lw + 16 * q < nws ? bt.lw + 16 * q : 0;
            const uint32_t *blk = kPanel ? xs + panel_block<B>(w) : xs + w * kBlk;
            dot_pair<B, kPanel>(v[2 * q], blk, (int)(bt.meta[q].x & 31u), (int)(bt.meta[q].y & 31u), acc);
            dot_pair<B, kPanel>(v[2 * q + 1], blk, (int)(bt.meta[q].z & 31u), (int)(bt.meta[q].w & 31u), acc);
        }
    } else if constexpr (B == 1) {
        constexpr int kCol = 2;  // LDS bytes of one column
        const bool odd = threadIdx.x & 1;
        const int wa = odd ? bt.lw - 32 : bt.lw, wb = wa + 32;  // words i and 32+i of the strip
        const bool oka = wa < nws, okb = wb < nws;
        const uint8_t *x8 = reinterpret_cast<const uint8_t *>(xs);
        const int ba = (oka ? wa : 0) * kBlk * 4, bb = (okb ? wb : 0) * kBlk * 4;  // block byte offsets
        // value pair k of the walk: even lanes dword k of a chunk; odd lanes dword 3 - k
        // with its halves swapped (the downward walk meets the higher column first)
        const uint32_t vsel = odd ? 0x01000302u : 0x07060504u;
        const uint32_t av[4] = {bt.va.x, bt.va.y, bt.va.z, bt.va.w}, bv[4] = {bt.vb.x, bt.vb.y, bt.vb.z, bt.vb.w};
        if constexpr (FMT == kMetaBitmask) {
            const uint32_t own = bt.meta[0].x, oth = pair_swap(own);
            uint32_t ma = odd ? oth : own, mb = odd ? own : oth;
            ma = oka && __builtin_popcount(ma) == 16 ? ma : 0xFFFFu;
            mb = okb && __builtin_popcount(mb) == 16 ? mb : 0xFFFFu;
            ma = odd ? __builtin_bitreverse32(ma) : ma;
            mb = odd ? __builtin_bitreverse32(mb) : mb;
            // byte address of the column at walk position p: base + dir * p (odd lanes: column 31 - p)
            const int dir = odd ? -kCol : kCol, flip = odd ? 31 * kCol : 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int a0 = __builtin_ctz(ma);
                ma &= ma - 1;
                const int a1 = __builtin_ctz(ma);
                ma &= ma - 1;
                const int b0 = __builtin_ctz(mb);
                mb &= mb - 1;
                const int b1 = __builtin_ctz(mb);
                mb &= mb - 1;
                dot_pair_at(__builtin_amdgcn_perm(av[k], av[3 - k], vsel), x8 + ba + flip + dir * a0,
                            x8 + ba + flip + dir * a1, acc[0]);
                dot_pair_at(__builtin_amdgcn_perm(bv[k], bv[3 - k], vsel), x8 + bb + flip + dir * b0,
                            x8 + bb + flip + dir * b1, acc[0]);
            }
        } else {
            // offsets of the lane's eight values of each word: even lanes bytes 0..7 of
            // words i (own) and 32+i (partner's); odd lanes bytes 8..15 of word i (partner's)
            // and of 32+i (own), then byte-reversed so that byte 2k is the walk's first
            const u32x4 own = bt.meta[0];
            const uint32_t r0 = pair_swap(odd ? own.x : own.z), r1 = pair_swap(odd ? own.y : own.w);
            const uint32_t a0 = odd ? r0 : own.x, a1 = odd ? r1 : own.y;
            const uint32_t b0 = odd ? own.z : r0, b1 = odd ? own.w : r1;
            const uint32_t rsel = odd ? 0x00010203u : 0x07060504u;  // odd: the other dword, bytes reversed
            const uint32_t oa[2] = {__builtin_amdgcn_perm(a0, a1, rsel), __builtin_amdgcn_perm(a1, a0, rsel)};
            const uint32_t ob[2] = {__builtin_amdgcn_perm(b0, b1, rsel), __builtin_amdgcn_perm(b1, b0, rsel)};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t pa = oa[k >> 1] >> (16 * (k & 1)), pb = ob[k >> 1] >> (16 * (k & 1));
                dot_pair_at(__builtin_amdgcn_perm(av[k], av[3 - k], vsel), x8 + ba + kCol * (int)(pa & 31u),
                            x8 + ba + kCol * (int)((pa >> 8) & 31u), acc[0]);
                dot_pair_at(__builtin_amdgcn_perm(bv[k], bv[3 - k], vsel), x8 + bb + kCol * (int)(pb & 31u),
                            x8 + bb + kCol * (int)((pb >> 8) & 31u), acc[0]);
            }
        }
    } else {
        const bool ok = bt.lw < nws;
        // Reassemble this lane's 16 values: even lanes keep their first chunk and receive
        // the partner's first chunk; odd lanes receive the partner's second chunk and keep
        // their own second chunk.
        const bool odd = threadIdx.x & 1;
        const uint32_t s_x = odd ? bt.va.x : bt.vb.x, s_y = odd ? bt.va.y : bt.vb.y;
        const uint32_t s_z = odd ? bt.va.z : bt.vb.z, s_w = odd ? bt.va.w : bt.vb.w;
        const uint32_t r_x = pair_swap(s_x), r_y = pair_swap(s_y), r_z = pair_swap(s_z), r_w = pair_swap(s_w);
        const uint32_t v[8] = {odd ? r_x : bt.va.x, odd ? r_y : bt.va.y, odd ? r_z : bt.va.z, odd ? r_w : bt.va.w,
                               odd ? bt.vb.x : r_x, odd ? bt.vb.y : r_y, odd ? bt.vb.z : r_z, odd ? bt.vb.w : r_w};
        // this word's 32 columns: word bt.lw is the lane's own word of its strip, so its
        // panel and stripe follow from the lane (panel_block for that word, without the
        // per-batch arithmetic); a lane past the slice reads block 0 (staged, finite x)
        using P = XPanel<B>;
        const int ln = threadIdx.x & (kWave - 1);
        const uint32_t *blk = ok ? xs + ((bt.lw >> 6) * P::kColDw + ln / P::kGroup) * P::kPanelDw + (ln % P::kGroup) * P::kColDw
                                 : xs;
        uint32_t mm = ok && __builtin_popcount(bt.meta[0].x) == 16 ? bt.meta[0].x : 0xFFFFu;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            int c0, c1;
            if constexpr (FMT == kMetaBitmask) {
                c0 = __builtin_ctz(mm);
                mm &= mm - 1;
                c1 = __builtin_ctz(mm);
                mm &= mm - 1;
            } else {
                const uint32_t o = bt.meta[0][k >> 1] >> (16 * (k & 1));  // offsets 2k, 2k+1
                c0 = (int)(o & 31u);
                c1 = (int)((o >> 8) & 31u);
            }
            dot_pair<B, kPanel>(v[k], blk, c0, c1, acc);
        }
    }
}

// Matrix and row within it of launch row r.
template <int EPI>
__device__ __forceinline__ void locate(const SpmvSet &set, int r, int &p, int &local) {
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

// Token whose row total lane `lane` holds after wave_sum_tokens<B> (2 <= B <= 4): lanes
// 0..3 hold tokens 0, 2, 1, 3 at B = 3-4, lanes 0..1 tokens 0, 1 at B = 2 (and every
// further lane repeats the pattern of its lane % 4).
template <int B>
__device__ __forceinline__ int token_of_lane(int lane) {
    return B == 2 ? (lane & 1) : 2 * (lane & 1) + ((lane >> 1) & 1);
}

// Row totals of B = 2..4 tokens at once: the first exchanges halve the tokens per lane
// (lane pairs swap half of their partial sums, then lane pairs two apart), so each lane
// adds one token's partials from then on: rotations by 4 and 8 within each 16-lane row
// and the cross-row sum.  Lane i ends with the total of token token_of_lane<B>(i); a
// fixed order of additions, so the result does not depend on timing.  The partial sums
// are cleared.
template <int B>
__device__ __forceinline__ float wave_sum_tokens(float (&a)[B], int lane) {
    static_assert(B >= 2 && B <= 4, "two to four tokens");
    auto dpp = [](float v, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xF, 0xF, false));
    };
    using X1 = std::integral_constant<int, 0xB1>;   // quad_perm(1,0,3,2): lane ^ 1
    using X2 = std::integral_constant<int, 0x4E>;   // quad_perm(2,3,0,1): lane ^ 2
    using R4 = std::integral_constant<int, 0x124>;  // row_ror:4
    using R8 = std::integral_constant<int, 0x128>;  // row_ror:8
    const bool odd = lane & 1;
    float c;
    if constexpr (B == 2) {
        c = (odd ? a[1] : a[0]) + dpp(odd ? a[0] : a[1], X1{});  // even lanes token 0, odd lanes token 1
        c = c + dpp(c, X2{});
    } else {
        float t3 = 0.f;
        if constexpr (B == 4) t3 = a[B - 1];
        // even lanes keep tokens 0 and 1, odd lanes 2 and 3
        const float b0 = (odd ? a[2] : a[0]) + dpp(odd ? a[0] : a[2], X1{});
        const float b1 = (odd ? t3 : a[1]) + dpp(odd ? a[1] : t3, X1{});
        const bool hi = lane & 2;  // lanes 2, 3 of a quad keep the second of the two
        c = (hi ? b1 : b0) + dpp(hi ? b0 : b1, X2{});
    }
#pragma unroll
    for (int b = 0; b < B; ++b) a[b] = 0.f;
    c = c + dpp(c, R4{});
    c = c + dpp(c, R8{});
    return cross_rows_sum(c);
}

// Row finished: wave reduction (uniform across the wave), then one lane per token writes
// the output -- the bf16 row; for the gated MLP h = silu(g) * u once the up row of a
// pair is done, the gate total kept in gsave until then; for a split launch the row's
// fp32 partial.  At one token and at 5..8 lane 0 writes every token; at 2..4 tokens the
// totals come from wave_sum_tokens and lanes 0..B-1 (B = 2) or 0..3 (B = 3-4; lane 3 has
// no token at B = 3) each write their own token (gsave[0] holds that token's gate total).
// `split` (0 or 1) and the row parity are integers: a boolean here would be materialised
// through a vector register, and the reuse of that register can make the wave wait for
// its in-flight loads.
template <int B, int EPI>
__device__ __forceinline__ void finish_row(float (&acc)[B], float (&gsave)[B], const SpmvSet &set, int row, int split,
                                           int s, int R, int lane, float *partial) {
    const int glu = EPI == kEpiSwiGLU ? 1 - split : 0;  // gated MLP without a split
    const int up = row & 1;
    if constexpr (B >= 2 && B <= 4) {
        const float tot = wave_sum_tokens<B>(acc, lane);
        float val = tot;
        if constexpr (EPI == kEpiSwiGLU) {
            gsave[0] = up ? gsave[0] : tot;
            val = glu ? silu_mul(gsave[0], tot) : tot;
        }
        const int t = token_of_lane<B>(lane);
        if ((glu & (up ^ 1)) | (lane >= (B == 2 ? 2 : 4)) | (t >= B)) return;
        if (split) {
            partial[((int64_t)s * B + t) * R + row] = val;
            return;
        }
        int p, local;
        locate<EPI>(set, row, p, local);
        set.y[p][(int64_t)t * set.ldy[p] + local] = f32_to_bf16_rne(val);
        return;
    }
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
        for (int b = 0; b < B; ++b) partial[((int64_t)s * B + b) * R + row] = val[b];
        return;
    }
    int p, local;
    locate<EPI>(set, row, p, local);
#pragma unroll
    for (int b = 0; b < B; ++b) set.y[p][(int64_t)b * set.ldy[p] + local] = f32_to_bf16_rne(val[b]);
}

// Batch loads of launch row r, word offset `base` within the slice.  meta0 / values0 are
// matrix 0's arrays as kernel arguments: a one-matrix launch reads only those, and the
// gated MLP picks between them and matrix 1's at a fixed argument offset, so neither
// waits for an argument load that depends on another before its first batch goes out.
template <int FMT, int EPI>
__device__ __forceinline__ void load_row_batch(Batch<FMT> &bt, const SpmvSet &set, const void *meta0,
                                               const uint16_t *values0, int r, int KW, int w0, int words, int base,
                                               int lane) {
    int p, local;
    locate<EPI>(set, r, p, local);
    const int64_t off = (int64_t)local * KW + w0;  // in words
    const void *mp;
    const uint16_t *vp;
    if constexpr (EPI == kEpiOne) {
        mp = meta0;
        vp = values0;
    } else if constexpr (EPI == kEpiSwiGLU) {
        mp = p ? set.meta[1] : meta0;
        vp = p ? set.values[1] : values0;
    } else {
        mp = set.meta[p];
        vp = set.values[p];
    }
    load_batch<FMT>(bt, reinterpret_cast<const uint8_t *>(mp) + off * meta_bytes(FMT),
                    reinterpret_cast<const u32x4 *>(vp) + off * 2, words, base, lane);
}

// The scalars that the first batch of loads depends on lead the argument list (matrix 0's
// arrays, the launch's row count R, the words per row KW, the grid width gx and whether
// rows are split): the library is built to preload leading kernel arguments into scalar
// registers, so a wave can issue its first weight loads without waiting for an argument
// load, and no dispatch-packet read is needed for the grid size.
template <int FMT, int B, int NT, int EPI>
__global__ __launch_bounds__(NT, NT == 1024 ? 8 : 1) void spmv_kernel(const void *meta0, const uint16_t *values0, int R,
                                                                      int KW, int gx, int split,
                                                                      const uint16_t *__restrict__ x, int64_t ldx,
                                                                      int slice, float *__restrict__ partial,
                                                                      const SpmvSet set) {
    extern __shared__ uint32_t xs[];  // x: [nws][XLayout<1>::kBlk] at one token, else whole strips of panels
    const int s = blockIdx.y;
    const int w0 = s * slice;
    const int nws = min(slice, KW - w0);
    const int lane = threadIdx.x & (kWave - 1);
    // wave-uniform by construction; readfirstlane lets the compiler keep the row loop
    // in scalar registers and branch on it without exec masking
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    constexpr int kWaves = NT / kWave;

    // This wave's rows: first_row, first_row + row_step, ... (gated MLP: the row pairs
    // 2i, 2i+1 for i = first pair, first pair + pair step, ...); each row slice is cut
    // into nb strips of 64 words, walked as one flat sequence so the next strip's loads
    // are in flight while the current one is computed, across row boundaries too.
    const int unit = blockIdx.x * kWaves + wave;
    const int row_step = gx * kWaves;
    const int first_row = EPI == kEpiSwiGLU ? 2 * unit : unit;
    const int units = EPI == kEpiSwiGLU ? R / 2 : R;
    const int my_rows = (unit < units ? (units - 1 - unit) / row_step + 1 : 0) * (EPI == kEpiSwiGLU ? 2 : 1);
    const int nb = (nws + kWave - 1) / kWave;
    const int total = my_rows * nb;
    auto next_row = [&](int r) {
        if constexpr (EPI == kEpiSwiGLU) return (r & 1) ? r - 1 + 2 * row_step : r + 1;
        return r + row_step;
    };

    // Two batch buffers used in turn: the loads of the next batch go out before the walk
    // of the current one.  No register copies, so the wait for one batch never covers
    // the loads of the other.
    Batch<FMT> bufA, bufB;
    auto step = [&](int &row, int &bi) {
        if (++bi == nb) {
            bi = 0;
            row = next_row(row);
        }
    };
    int rowA = first_row, biA = 0, rowB = first_row, biB = 0;
    // Stage this slice of x into LDS; batch 0's loads go out right after the first round
    // of x loads, so waiting for x (an L2 hit after the first workgroup of an XCD) never
    // waits for the weights queued behind it.
    stage_x<B, NT, (B >= 2)>(xs, x, ldx, w0, nws, [&] {
        load_row_batch<FMT, EPI>(bufA, set, meta0, values0, min(rowA, R - 1), KW, w0, total > 0 ? nws : 0, 0, lane);
    });
    __syncthreads();

    float acc[B], gsave[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = gsave[b] = 0.f;
    // Whole pairs of batches per iteration and the odd last batch after the loop: an exit
    // in the middle of the body would give the wait-count analysis a path back to the
    // top with a batch's loads still in flight, and it would then wait for them there.
    // The loads are unconditional (a conditional load makes every later wait a full
    // one); the one batch past the end, when the count is even, has zero words -- no
    // memory traffic -- and goes out before the last walk, which hides its round trip.
    int t = 0;
    for (; t + 1 < total; t += 2) {
        rowB = rowA;
        biB = biA;
        step(rowB, biB);
        load_row_batch<FMT, EPI>(bufB, set, meta0, values0, min(rowB, R - 1), KW, w0, nws, biB * kWave, lane);  // batch t+1
        // keep the walk (which waits for batch A) after the issue of these loads
        __builtin_amdgcn_sched_barrier(0);
        walk_batch<FMT, B>(bufA, xs, nws, acc);  // batch t
        if (biA == nb - 1) finish_row<B, EPI>(acc, gsave, set, rowA, split, s, R, lane, partial);
        rowA = rowB;
        biA = biB;
        step(rowA, biA);
        load_row_batch<FMT, EPI>(bufA, set, meta0, values0, min(rowA, R - 1), KW, w0, t + 2 < total ? nws : 0, biA * kWave, lane);
        __builtin_amdgcn_sched_barrier(0);
        walk_batch<FMT, B>(bufB, xs, nws, acc);  // batch t+1
        if (biB == nb - 1) finish_row<B, EPI>(acc, gsave, set, rowB, split, s, R, lane, partial);
    }
    if (t < total) {  // odd count: the last batch is in A
        walk_batch<FMT, B>(bufA, xs, nws, acc);
        if (biA == nb - 1) finish_row<B, EPI>(acc, gsave, set, rowA, split, s, R, lane, partial);
    }
}

// Half-row walk (one matrix, bitmask, one token; rows of at least 7 strips, one row per
// wave pair).  The 16 waves of a workgroup cover 8 rows: wave w walks the first (w < 8)
// or the second half of the strips of row blockIdx.x * 8 + w % 8, so a CU holds twice the
// waves it would with one row per wave and each wave's chain of strips is half as long.
// The halves' totals meet in LDS without a barrier: lane 0 of each wave stores its total
// and then increments the row's counter (workgroup-scope release/acquire); the second to
// arrive adds the two totals in half order (deterministic) and stores the row.
constexpr int kHalfThreads = 1024;
constexpr int kHalfRows = kHalfThreads / kWave / 2;  // rows per workgroup

template <int B, int EPI>
__global__ __launch_bounds__(kHalfThreads, 8) void spmv_half_kernel(const void *meta0, const uint16_t *values0, int R,
                                                                    int KW, const uint16_t *__restrict__ x,
                                                                    int64_t ldx, const SpmvSet set) {
    static_assert(EPI == kEpiOne && B == 1, "one matrix and one token per launch (blocked x)");
    extern __shared__ uint32_t xs[];  // x [KW][kBlk], then totals [rows][2][B], then counters [rows]
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int half = wave / kHalfRows, rl = wave - half * kHalfRows;
    const int nb = (KW + kWave - 1) / kWave, h0 = (nb + 1) / 2;
    const int first = half ? h0 : 0, ns = half ? nb - h0 : h0;  // this wave's strips
    const int row = blockIdx.x * kHalfRows + rl;
    const int live = row < R ? KW : 0;  // words to load: none for rows past the matrix
    const int rr = min(row, R - 1);
    float *tot = reinterpret_cast<float *>(xs + (size_t)KW * XLayout<B>::kBlk);
    uint32_t *cnt = reinterpret_cast<uint32_t *>(tot + kHalfRows * 2 * B);
    if ((int)threadIdx.x < kHalfRows) cnt[threadIdx.x] = 0u;

    Batch<kMetaBitmask> bufA, bufB;
    stage_x<B, kHalfThreads>(xs, x, ldx, 0, KW, [&] {
        load_row_batch<kMetaBitmask, EPI>(bufA, set, meta0, values0, rr, KW, 0, live, first * kWave, lane);
    });
    __syncthreads();
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;
    // two buffers in turn, whole pairs in the loop and the odd last strip after it, as in
    // spmv_kernel; the strip loaded past this half has no words (no memory traffic)
    int t = 0;
    for (; t + 1 < ns; t += 2) {
        load_row_batch<kMetaBitmask, EPI>(bufB, set, meta0, values0, rr, KW, 0, live, (first + t + 1) * kWave, lane);
        __builtin_amdgcn_sched_barrier(0);
        walk_batch<kMetaBitmask, B>(bufA, xs, KW, acc);
        load_row_batch<kMetaBitmask, EPI>(bufA, set, meta0, values0, rr, KW, 0, t + 2 < ns ? live : 0,
                                          (first + t + 2) * kWave, lane);
        __builtin_amdgcn_sched_barrier(0);
        walk_batch<kMetaBitmask, B>(bufB, xs, KW, acc);
    }
    if (t < ns) walk_batch<kMetaBitmask, B>(bufA, xs, KW, acc);
    float v[B];
#pragma unroll
    for (int b = 0; b < B; ++b) v[b] = wave_sum(acc[b]);
    if (lane != 0 || row >= R) return;
#pragma unroll
    for (int b = 0; b < B; ++b) tot[(rl * 2 + half) * B + b] = v[b];
    const uint32_t prev = __hip_atomic_fetch_add(&cnt[rl], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (prev != 1u) return;  // the other half is still walking: it stores the row
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const float o = tot[(rl * 2 + (half ^ 1)) * B + b];
        set.y[0][(int64_t)b * set.ldy[0] + row] = f32_to_bf16_rne(half ? o + v[b] : v[b] + o);
    }
}

// Strip walk (one matrix, bitmask, one token).  A workgroup of NT threads owns rpw
// consecutive rows; their strips, taken row by row as one sequence, are dealt to the
// waves in turn (wave w walks strips w, w + W, w + 2W, ... of the sequence), so every
// wave of every workgroup has the same number of strips to within one whatever R, and the
// W waves of a workgroup read W adjacent pieces of one contiguous stretch of the matrix
// at about the same time.  Each strip's total (a wave reduction) goes to LDS; after a
// barrier every row adds its strips in strip order (deterministic) and stores.  The
// planner takes it where whole rows or half rows per wave would leave the CUs unevenly
// loaded, or for long matrices of rows of few strips.
template <int B, int EPI, int NT>
__global__ __launch_bounds__(NT, NT == 1024 ? 8 : 1) void spmv_strip_kernel(const void *meta0, const uint16_t *values0,
                                                                            int R, int KW, int rpw,
                                                                            const uint16_t *__restrict__ x,
                                                                            int64_t ldx, const SpmvSet set) {
    static_assert(EPI == kEpiOne && B == 1, "one matrix and one token per launch (blocked x)");
    constexpr int W = NT / kWave;
    extern __shared__ uint32_t xs[];  // x [KW][kBlk], then strip totals [rpw * nb][B]
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nb = (KW + kWave - 1) / kWave;
    const int r0 = blockIdx.x * rpw;
    const int nr = min(rpw, R - r0);  // >= 1: the grid is ceil(R / rpw)
    const int T = nr * nb;            // strips of this workgroup
    float *part = reinterpret_cast<float *>(xs + (size_t)KW * XLayout<B>::kBlk);
    const int n = T > wave ? (T - 1 - wave) / W + 1 : 0;  // strips of this wave
    // strip j of the sequence is strip j % nb of row r0 + j / nb; a step of W strips
    // moves dq rows and dr strips
    const int dq = W / nb, dr = W - dq * nb;
    auto advance = [&](int &r, int &s) {
        s += dr;
        r += dq;
        if (s >= nb) {
            s -= nb;
            ++r;
        }
    };
    int rowA = r0 + wave / nb, sA = wave - (wave / nb) * nb, jA = wave;
    int rowB = rowA, sB = sA, jB = jA;
    Batch<kMetaBitmask> bufA, bufB;
    stage_x<B, NT>(xs, x, ldx, 0, KW, [&] {
        load_row_batch<kMetaBitmask, EPI>(bufA, set, meta0, values0, min(rowA, R - 1), KW, 0, n > 0 ? KW : 0,
                                          sA * kWave, lane);
    });
    __syncthreads();
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.f;
    auto strip_done = [&](int j) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float tsum = wave_sum(acc[b]);
            acc[b] = 0.f;
            if (lane == 0) part[j * B + b] = tsum;
        }
    };
    // two buffers in turn, whole pairs in the loop and the odd last strip after it, as in
    // spmv_kernel; the strip loaded past this wave's last has no words (no memory traffic)
    int t = 0;
    for (; t + 1 < n; t += 2) {
        rowB = rowA;
        sB = sA;
        advance(rowB, sB);
        jB = jA + W;
        load_row_batch<kMetaBitmask, EPI>(bufB, set, meta0, values0, min(rowB, R - 1), KW, 0, KW, sB * kWave, lane);
        __builtin_amdgcn_sched_barrier(0);
        walk_batch<kMetaBitmask, B>(bufA, xs, KW, acc);
        strip_done(jA);
        rowA = rowB;
        sA = sB;
        advance(rowA, sA);
        jA = jB + W;
        load_row_batch<kMetaBitmask, EPI>(bufA, set, meta0, values0, min(rowA, R - 1), KW, 0, t + 2 < n ? KW : 0,
                                          sA * kWave, lane);
        __builtin_amdgcn_sched_barrier(0);
        walk_batch<kMetaBitmask, B>(bufB, xs, KW, acc);
        strip_done(jB);
    }
    if (t < n) {
        walk_batch<kMetaBitmask, B>(bufA, xs, KW, acc);
        strip_done(jA);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nr * B; i += NT) {
        const int rl = i / B, b = i - rl * B;
        float s = 0.f;
        for (int k = 0; k < nb; ++k) s += part[(rl * nb + k) * B + b];
        set.y[0][(int64_t)b * set.ldy[0] + r0 + rl] = f32_to_bf16_rne(s);
    }
}

// Second pass of split rows: add the slices in order, round once to bf16.
template <int B>
__global__ __launch_bounds__(256) void split_finish_kernel(const float *__restrict__ partial, int S,
                                                           const SpmvSet set) {
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

// The same for the gated MLP: gate and up totals of row i (launch rows 2i, 2i+1).
template <int B>
__global__ __launch_bounds__(256) void split_finish_swiglu_kernel(const float *__restrict__ partial, int S,
                                                                  const SpmvSet set) {
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

// Raise the dynamic-LDS limit of one kernel instance once per device.
template <int FMT, int B, int NT, int EPI>
hipError_t allow_lds(size_t bytes) {
    static std::atomic<uint64_t> done{0};
    if (bytes <= 64 * 1024) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = 1ull << (dev & 63);
    if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
    e = hipFuncSetAttribute((const void *)spmv_kernel<FMT, B, NT, EPI>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kLdsCap);
    if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

template <int FMT, int B, int NT, int EPI>
hipError_t launch_fbn(const MvPlan &p, const SpmvSet &set, int64_t K, const uint16_t *x, int64_t ldx, float *ws,
                      hipStream_t st) {
    hipError_t e = allow_lds<FMT, B, NT, EPI>(p.lds_bytes);
    if (e != hipSuccess) return e;
    SpmvSet padded = set;
    for (int q = set.P + 1; q <= kMaxMats; ++q) padded.row0[q] = set.row0[set.P];
    hipLaunchKernelGGL((spmv_kernel<FMT, B, NT, EPI>), dim3(p.grid_x, p.splits), dim3(NT), p.lds_bytes, st,
                       set.meta[0], set.values[0], set.row0[set.P], (int)(K / 32), p.grid_x, p.splits > 1 ? 1 : 0, x,
                       ldx, p.slice, ws, padded);
    e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    const int R = set.row0[set.P];
    if constexpr (EPI == kEpiSwiGLU)
        hipLaunchKernelGGL(split_finish_swiglu_kernel<B>, dim3((unsigned)((R / 2 + 255) / 256)), dim3(256), 0, st,
                           ws, p.splits, set);
    else
        hipLaunchKernelGGL(split_finish_kernel<B>, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, st, ws,
                           p.splits, set);
    return hipGetLastError();
}

template <int B>
hipError_t launch_half(const MvPlan &p, const SpmvSet &set, int64_t K, const uint16_t *x, int64_t ldx,
                       hipStream_t st) {
    static std::atomic<uint64_t> done{0};
    if (p.lds_bytes > 64 * 1024) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        const uint64_t bit = 1ull << (dev & 63);
        if (!(done.load(std::memory_order_acquire) & bit)) {
            e = hipFuncSetAttribute((const void *)spmv_half_kernel<B, kEpiOne>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsCap);
            if (e != hipSuccess) return e;
            done.fetch_or(bit, std::memory_order_acq_rel);
        }
    }
    hipLaunchKernelGGL((spmv_half_kernel<B, kEpiOne>), dim3(p.grid_x), dim3(kHalfThreads), p.lds_bytes, st,
                       set.meta[0], set.values[0], set.row0[set.P], (int)(K / 32), x, ldx, set);
    return hipGetLastError();
}

template <int B, int NT>
hipError_t launch_strip(const MvPlan &p, const SpmvSet &set, int64_t K, const uint16_t *x, int64_t ldx,
                        hipStream_t st) {
    static std::atomic<uint64_t> done{0};
    if (p.lds_bytes > 64 * 1024) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        const uint64_t bit = 1ull << (dev & 63);
        if (!(done.load(std::memory_order_acquire) & bit)) {
            e = hipFuncSetAttribute((const void *)spmv_strip_kernel<B, kEpiOne, NT>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsCap);
            if (e != hipSuccess) return e;
            done.fetch_or(bit, std::memory_order_acq_rel);
        }
    }
    hipLaunchKernelGGL((spmv_strip_kernel<B, kEpiOne, NT>), dim3(p.grid_x), dim3(NT), p.lds_bytes, st, set.meta[0],
                       set.values[0], set.row0[set.P], (int)(K / 32), p.rows_per_group, x, ldx, set);
    return hipGetLastError();
}

template <int FMT, int B, int EPI>
hipError_t launch_fb(const MvPlan &p, const SpmvSet &set, int64_t K, const uint16_t *x, int64_t ldx, float *ws,
                     hipStream_t st) {
    if constexpr (FMT == kMetaBitmask && B == 1 && EPI == kEpiOne)
        if (p.walk != kWalkRows) {
            if (p.walk == kWalkHalf) return launch_half<B>(p, set, K, x, ldx, st);
            if (p.walk == kWalkStrips && p.threads == 1024) return launch_strip<B, 1024>(p, set, K, x, ldx, st);
            if (p.walk == kWalkStrips && p.threads == 512) return launch_strip<B, 512>(p, set, K, x, ldx, st);
        }
    if (p.walk != kWalkRows) return hipErrorInvalidValue;
    if constexpr (wide_ok(FMT, B))
        if (p.threads == 1024) return launch_fbn<FMT, B, 1024, EPI>(p, set, K, x, ldx, ws, st);
    if (p.threads == 256) return launch_fbn<FMT, B, 256, EPI>(p, set, K, x, ldx, ws, st);
    return launch_fbn<FMT, B, 512, EPI>(p, set, K, x, ldx, ws, st);
}

template <int FMT, int EPI>
hipError_t launch_f(const MvPlan &p, const SpmvSet &set, int64_t K, const uint16_t *x, int64_t ldx, int B, float *ws,
                    hipStream_t st) {
    switch (B) {
    case 1: return launch_fb<FMT, 1, EPI>(p, set, K, x, ldx, ws, st);
    case 2: return launch_fb<FMT, 2, EPI>(p, set, K, x, ldx, ws, st);
    case 3: return launch_fb<FMT, 3, EPI>(p, set, K, x, ldx, ws, st);
    case 4: return launch_fb<FMT, 4, EPI>(p, set, K, x, ldx, ws, st);
    case 5: return launch_fb<FMT, 5, EPI>(p, set, K, x, ldx, ws, st);
    case 6: return launch_fb<FMT, 6, EPI>(p, set, K, x, ldx, ws, st);
    case 7: return launch_fb<FMT, 7, EPI>(p, set, K, x, ldx, ws, st);
    case 8: return launch_fb<FMT, 8, EPI>(p, set, K, x, ldx, ws, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t spmv_lds_per_word(int B) { return (size_t)blk_dwords(B) * 4; }

// x of the N:M word walk: blocked at one token; at two or more tokens the panel layout,
// 64*S bytes per word in whole 64-word strips (S = 2, 4 or 8 token slots per column).
static size_t spmv_x_bytes_per_word(int B) { return B == 1 ? (size_t)blk_dwords(1) * 4 : (size_t)64 * (B <= 2 ? 2 : B <= 4 ? 4 : 8); }
static size_t spmv_x_lds_bytes(int64_t nws, int B) {
    return spmv_x_bytes_per_word(B) * (size_t)(B == 1 ? nws : (nws + kWave - 1) / kWave * kWave);
}

// Device-resident scratch of the no-allocation entry point: the fp32 partial sums of split
// rows, in a fixed array of kSpmvScratchBytes on every device the library runs on (held
// until the process ends).  In host code `scratch` only names the symbol; its device
// address comes from hipGetSymbolAddress, looked up once per device with that device
// current and kept per device, and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[kSpmvScratchBytes];

hipError_t spmv_scratch(void **ptr) {
    static std::mutex mu;
    static void *addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

MvPlan plan_spmv(int64_t R, int64_t K, int B, const DeviceInfo &dev, int fmt) {
    MvPlan p;
    p.threads = kThreads;
    const int64_t KW = K / 32;
    const int64_t bytes_per_word = (int64_t)spmv_x_bytes_per_word(B);
    size_t cap = kLdsCap;
    if (dev.max_lds_per_block > 0 && (size_t)dev.max_lds_per_block < cap) cap = (size_t)dev.max_lds_per_block;
    int64_t max_slice = (int64_t)cap / bytes_per_word;
    if (max_slice >= kWave) max_slice -= max_slice % kWave;
    if (max_slice < 1) max_slice = 1;
    // Split rows across workgroups only when LDS cannot hold a row's x, or when the
    // matrix has too few rows to give every CU a couple of waves: the split costs a
    // second launch, which outweighs the extra parallelism on anything but very short,
    // wide matrices.  No slice is shorter than one 64-word strip.
    const int64_t cu = dev.num_cu > 0 ? dev.num_cu : 256;
    const int64_t want_rows = cu * 2;
    int64_t splits = (KW + max_slice - 1) / max_slice;
    int64_t by_tasks = R >= want_rows ? 1 : (want_rows + R - 1) / R;
    int64_t max_by_len = KW / kWave > 0 ? KW / kWave : 1;
    if (by_tasks > max_by_len) by_tasks = max_by_len;
    if (splits < by_tasks) splits = by_tasks;
    int64_t slice = (KW + splits - 1) / splits;
    if (slice > kWave) slice = (slice + kWave - 1) / kWave * kWave;
    if (slice > max_slice) slice = max_slice;
    splits = (KW + slice - 1) / slice;
    p.splits = (int)splits;
    p.slice = (int)slice;
    p.lds_bytes = spmv_x_lds_bytes(slice, B);
    int per_cu = (int)(kLdsPerCu / (p.lds_bytes > 0 ? p.lds_bytes : 1));
    if (per_cu > 4) per_cu = 4;
    if (per_cu < 1) per_cu = 1;
    // Matrices with too few rows to give every CU a 512-thread workgroup use 256-thread
    // workgroups, which spreads them over twice as many CUs.
    if ((R + kThreads / kWave - 1) / (kThreads / kWave) * splits < cu)
        p.threads = 256;
    else if (per_cu <= 2 && wide_ok(fmt, B) && B >= 3)
        p.threads = 1024;  // x large enough to allow only two workgroups: twice the waves per CU
    else if (B <= 2 && wide_ok(fmt, B) && (per_cu <= 2 || (KW >= 256 && splits == 1))) {
        // Rows of 8192+ columns at B <= 2: two 16-wave workgroups per CU stage x half as
        // often as four 8-wave ones, where the larger workgroups still split evenly -- the
        // same number of rows for every wave and the same number of workgroups on every
        // CU (5120 rows: 320 workgroups on 256 CUs made the launch 10-14% slower).
        const int64_t g16 = std::min<int64_t>((R + 15) / 16, (2 * cu + splits - 1) / splits);
        if (R % (16 * g16) == 0 && (g16 * splits) % cu == 0) {
            p.threads = 1024;
            per_cu = 2;
        }
    }
    const int64_t waves = p.threads / kWave;
    int64_t gx = (R + waves - 1) / waves;
    int64_t cap_x = (per_cu * cu + splits - 1) / splits;
    if (gx > cap_x) gx = cap_x;
    if (gx < 1) gx = 1;
    p.grid_x = (int)gx;
    p.unroll = 1;
    p.ws_bytes = splits > 1 ? (size_t)splits * B * R * sizeof(float) : 0;
    return p;
}

MvPlan plan_spmv_one(const MvPlan &word, int64_t R, int64_t K, int B, const DeviceInfo &dev) {
    const int64_t cu = dev.num_cu > 0 ? dev.num_cu : 256;
    const int64_t KW = K / 32, nb = (KW + kWave - 1) / kWave;
    if (B != 1 || word.tile || word.splits != 1) return word;
    const size_t xb = (size_t)KW * spmv_lds_per_word(B);  // x of a whole row
    auto strips = [&](int threads, int64_t groups_per_cu) {
        const int64_t rpw = (R + groups_per_cu * cu - 1) / (groups_per_cu * cu);
        const size_t lds = xb + (size_t)rpw * nb * B * sizeof(float);
        if (lds * groups_per_cu > kLdsPerCu || lds > kLdsCap) return word;
        MvPlan p = word;
        p.walk = kWalkStrips;
        p.threads = threads;
        p.rows_per_group = (int)rpw;
        p.grid_x = (int)((R + rpw - 1) / rpw);
        p.lds_bytes = lds;
        return p;
    };
    if (nb >= 7 && R >= 2 * cu * kHalfRows) {
        // Rows of 7+ strips, at least 16 per CU.  Where the rows fill whole rounds of two
        // 16-wave workgroups per CU, split each row between two waves (8B down 4096 x
        // 14336: 12.61 -> 12.40 us; 70B down 8192 x 28672: 41.98 -> 41.41 us).  Otherwise
        // (5120 rows: 640 half-row workgroups, or 1.25 rows per wave) deal the strips of
        // 10 rows per workgroup to its 16 waves (Qwen3-14B down 5120 x 17408: 19.87 ->
        // 17.92 us; Qwen3-32B down 5120 x 25600: 26.42 -> 25.78 us).
        if (R % (2 * cu * kHalfRows) != 0) return strips(1024, 2);
        const size_t extra = (size_t)kHalfRows * 2 * B * 4 + kHalfRows * 4;
        if (R > (int64_t)word.grid_x * (word.threads / kWave) || word.lds_bytes + extra > kLdsCap) return word;
        MvPlan p = word;
        p.walk = kWalkHalf;
        p.threads = kHalfThreads;
        p.grid_x = (int)((R + kHalfRows - 1) / kHalfRows);
        p.lds_bytes = word.lds_bytes + extra;
        return p;
    }
    // Rows of 8192-12288 columns (4-6 strips) and at least 4 strips for every wave of four
    // 8-wave workgroups per CU: deal the strips of consecutive rows to the waves, which
    // then sweep one contiguous stretch of the matrix together (70B q 8192 x 8192: 14.15
    // -> 13.68 us; 70B gate 28672 x 8192: 42.61 -> 41.71 us).  Shorter rows keep whole
    // rows per wave: the strip walk was 1-9% slower on the 8B shapes.
    if (KW >= 256 && nb <= 6 && R * nb >= 4 * (4 * cu * (kThreads / kWave))) return strips(kThreads, 4);
    return word;
}

hipError_t launch_spmv(const MvPlan &p, const SpmvSet &set, int fmt, int64_t K, const uint16_t *x, int64_t ldx, int B,
                       float *ws, hipStream_t st) {
    switch (fmt) {
    case kMetaBitmask:
        return set.P == 1 ? launch_f<kMetaBitmask, kEpiOne>(p, set, K, x, ldx, B, ws, st)
                          : launch_f<kMetaBitmask, kEpiNone>(p, set, K, x, ldx, B, ws, st);
    case kMetaU8:
        return set.P == 1 ? launch_f<kMetaU8, kEpiOne>(p, set, K, x, ldx, B, ws, st)
                          : launch_f<kMetaU8, kEpiNone>(p, set, K, x, ldx, B, ws, st);
    case kMetaI32:
        return set.P == 1 ? launch_f<kMetaI32, kEpiOne>(p, set, K, x, ldx, B, ws, st)
                          : launch_f<kMetaI32, kEpiNone>(p, set, K, x, ldx, B, ws, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_spmv_swiglu(const MvPlan &p, const SpmvSet &set, int64_t K, const uint16_t *x, int64_t ldx, int B,
                              float *ws, hipStream_t st) {
    if (set.P != 2 || set.row0[2] != 2 * set.row0[1]) return hipErrorInvalidValue;
    return launch_f<kMetaBitmask, kEpiSwiGLU>(p, set, K, x, ldx, B, ws, st);
}

}  // namespace nmk
