// nm_kernels.h -- internal launch interface between the C ABI (api.cpp) and the
// gfx950 kernels.  Not installed; callers use include/nm_spmv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nmk {

struct DeviceInfo {
    int num_cu = 0;            // compute units on the current device
    int max_lds_per_block = 0; // bytes of LDS one workgroup may allocate
};

// Launch plan of the split-row matrix-vector kernels.  Each row's reduction range
// (mask words for the sparse kernel, 8-column chunks for the dense one) is cut into
// `splits` contiguous slices of at most `slice` units.  grid = (grid_x, splits);
// workgroup w of slice s stages that slice of x in LDS once and then walks rows
// w*waves + wave, stepping by grid_x*waves.  With splits > 1 the slices write fp32
// partial sums to the workspace and a second kernel adds them in slice order.
struct MvPlan {
    int splits = 1;
    int slice = 0;          // units per slice
    int grid_x = 1;
    int threads = 512;      // workgroup size
    int unroll = 1;         // dense kernel: 8-column chunks per lane and batch (1, 2 or 4); tile kernel: tiles per step
    size_t lds_bytes = 0;   // dynamic LDS per workgroup
    size_t ws_bytes = 0;    // workspace bytes (0 when splits == 1)
    int tile = 0;           // 1: the matrix-core tile kernel (nm_spmv_tile.hip), 16-row tiles (threads / 64 waves)
    int tiles = 0;          // tile kernel: number of units (16 or 32 rows; unroll = tiles per unit)
    int xreg = 0;           // tile kernel: steps per wave and unit whose x operand stays in registers (0: none)
    int walk = 0;           // one-token single-matrix walks (nm_spmv.hip): kWalkRows, kWalkHalf, kWalkStrips
    int rows_per_group = 0; // kWalkStrips: consecutive rows owned by one workgroup
};

// Word-per-lane walks of a launch.  kWalkRows: each wave walks whole rows (any batch
// size, any set of matrices).  kWalkHalf: one matrix, one token; each row is split
// between two waves of a 16-wave workgroup.  kWalkStrips: one matrix, one token; a
// workgroup owns consecutive rows and deals their strips to its waves in turn.
constexpr int kWalkRows = 0;
constexpr int kWalkHalf = 1;
constexpr int kWalkStrips = 2;

// Row epilogues of the matrix-vector kernels.  kEpiNone: every row's total is one
// output.  kEpiSwiGLU: the set is the gate (matrix 0) and up (matrix 1) projections of a
// gated MLP with R rows each; launch row 2i is gate row i and 2i+1 up row i, a wave walks
// the two back to back and writes h_i = silu(g_i) * u_i (fp32, one bf16 rounding) to
// matrix 0's output.
constexpr int kEpiNone = 0;
constexpr int kEpiSwiGLU = 1;
// kEpiOne: a launch over a single matrix (set.P == 1).  Same rows and outputs as kEpiNone;
// the matrix's pointers come straight from the kernel arguments, with no row-to-matrix
// lookup, so a wave can issue its first loads from preloaded argument registers.
constexpr int kEpiOne = 2;

// Matrices that read the same input x (q, k, v; gate, up) walked by one launch: global
// row r belongs to matrix p when row0[p] <= r < row0[p + 1]; x is staged once.
constexpr int kMaxMats = 8;

// Metadata formats of the sparse kernel (values of nm_meta_format): per 32-column word,
// a 32-bit mask, 16 uint8 offsets within the word, or 16 int32 column indices.
constexpr int kMetaBitmask = 0;
constexpr int kMetaU8 = 1;
constexpr int kMetaI32 = 2;

struct SpmvSet {
    int P = 0;
    int row0[kMaxMats + 1] = {};
    const void *meta[kMaxMats] = {};  // metadata in the launch's format
    const uint16_t *values[kMaxMats] = {};
    uint16_t *y[kMaxMats] = {};
    int64_t ldy[kMaxMats] = {};
};

struct DenseSet {
    int P = 0;
    int row0[kMaxMats + 1] = {};
    const uint16_t *W[kMaxMats] = {};
    int64_t ldw[kMaxMats] = {};
    uint16_t *y[kMaxMats] = {};
    int64_t ldy[kMaxMats] = {};
};

// fmt: the launchs metadata format (the planner picks 1024-thread workgroups only for
// kernels that fit them without spilling).
MvPlan plan_spmv(int64_t R, int64_t K, int B, const DeviceInfo &dev, int fmt = kMetaBitmask);
// The walk of a one-matrix bitmask launch: the half-row or the strip walk where one of
// them applies (one token, no split rows), else `word` as is.
MvPlan plan_spmv_one(const MvPlan &word, int64_t R, int64_t K, int B, const DeviceInfo &dev);
size_t spmv_lds_per_word(int B);  // LDS bytes of x per 32-column block, blocked layout (unstructured kernel)
// Fixed device scratch for callers that cannot allocate (nm_spmv_noalloc): its device
// address on the current device (looked up once per device), kSpmvScratchBytes long.
constexpr size_t kSpmvScratchBytes = (size_t)4 << 20;
hipError_t spmv_scratch(void **ptr);
// epi: the launch's epilogue, which decides whether the 1024-thread workgroup variant
// fits without spilling.
MvPlan plan_dense(int64_t R, int64_t K, int B, const DeviceInfo &dev, int epi = kEpiNone);

hipError_t launch_col_norm(const uint16_t *X, int64_t T, int64_t K, int64_t ldx, float *n, hipStream_t st);
hipError_t launch_prune_pack(const uint16_t *W, int64_t ldw, int64_t R, int64_t K, const float *n, int N, int M,
                             uint32_t *masks, uint16_t *values, hipStream_t st);
hipError_t launch_unpack(const uint32_t *masks, const uint16_t *values, int64_t R, int64_t K, uint16_t *W,
                         int64_t ldw, hipStream_t st);
// 50% unstructured rows (K/2 kept per row; same encoding, varying set bits per word).
hipError_t launch_prune_pack_unstructured(const uint16_t *W, int64_t ldw, int64_t R, int64_t K, const float *n,
                                         uint32_t *masks, uint16_t *values, hipStream_t st);
hipError_t launch_unpack_unstructured(const uint32_t *masks, const uint16_t *values, int64_t R, int64_t K,
                                      uint16_t *W, int64_t ldw, hipStream_t st);
MvPlan plan_spmv_unstructured(int64_t R, int64_t K, int B, const DeviceInfo &dev);
hipError_t launch_spmv_unstructured(const MvPlan &p, const uint32_t *masks, const uint16_t *values, int64_t R,
                                    int64_t K, const uint16_t *x, int64_t ldx, int B, uint16_t *y, int64_t ldy,
                                    float *ws, hipStream_t st);
// OBS / SparseGPT solver (fp64).  Workspace sizes in bytes.
size_t sparsegpt_factor_workspace(int64_t K);
size_t sparsegpt_workspace(int64_t R, int64_t K);
hipError_t launch_hessian(const uint16_t *X, int64_t T, int64_t K, int64_t ldx, double *H, int64_t ldh,
                          hipStream_t st);
hipError_t launch_inverse_factor(const double *H, int64_t ldh, int64_t K, double damp, double *U, int64_t ldu,
                                 void *ws, hipStream_t st);
hipError_t launch_sparsegpt(const uint16_t *W, int64_t ldw, int64_t R, int64_t K, const double *H, int64_t ldh,
                            int N, int M, double damp, uint32_t *masks, uint16_t *values, void *ws, hipStream_t st);
hipError_t launch_meta_from_mask(const uint32_t *masks, int64_t R, int64_t K, int fmt, void *meta, hipStream_t st);
// R of the plan = total rows of the set (set.row0[set.P]).
hipError_t launch_spmv(const MvPlan &p, const SpmvSet &set, int fmt, int64_t K, const uint16_t *x, int64_t ldx,
                       int B, float *ws, hipStream_t st);
// Gated MLP: set = {gate, up}, R rows each (row0 = {0, R, 2R}); y[0] receives
// silu(gate x) * (up x).  Plan for 2R rows.
hipError_t launch_spmv_swiglu(const MvPlan &p, const SpmvSet &set, int64_t K, const uint16_t *x, int64_t ldx, int B,
                              float *ws, hipStream_t st);
// Bitmask launches with B >= kTileMinB tokens run on the matrix cores: each 16-row tile
// of mask words is expanded into a dense tile in LDS and multiplied by the inputs with
// MFMA.  spmv_tile_ok says whether a set qualifies (K a multiple of 1024, matrices of a
// plain set starting at multiples of 16 rows, 32-bit buffer ranges); the tile plan needs
// no workspace.  R = rows of the launch (gated MLP: 2 x the rows of each matrix).  With
// kTileLowB <= B < kTileMinB the tile kernel is taken only where the word-per-lane
// kernel would cut K into slices (a row's x too large for LDS): it reads x from L2 and
// needs neither the partial sums nor the second pass.
constexpr int kTileMinB = 5;
constexpr int kTileLowB = 3;
bool spmv_tile_ok(const SpmvSet &set, int64_t K, int64_t ldx, int B, int fmt, int epi);
MvPlan plan_spmv_tile(const SpmvSet &set, int64_t K, int B, const DeviceInfo &dev, int epi);
hipError_t launch_spmv_tile(const MvPlan &p, const SpmvSet &set, int64_t K, const uint16_t *x, int64_t ldx, int B,
                            int epi, hipStream_t st);
hipError_t launch_dense(const MvPlan &p, const DenseSet &set, int64_t K, const uint16_t *x, int64_t ldx, int B,
                        float *ws, hipStream_t st);
hipError_t launch_dense_swiglu(const MvPlan &p, const DenseSet &set, int64_t K, const uint16_t *x, int64_t ldx, int B,
                               float *ws, hipStream_t st);
// Measurement aid: one streaming read of `bytes` bytes (multiple of 16, <= 2^31), one
// XOR-fold per wave into sink[0 .. stream_read_waves(bytes)).
size_t stream_read_groups(size_t bytes);
size_t stream_read_waves(size_t bytes);
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st);

}  // namespace nmk
