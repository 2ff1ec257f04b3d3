// api.cpp -- the C ABI of include/nm_spmv.h: argument validation, error reporting,
// per-device properties and kernel dispatch.  Every argument check runs before the
// first HIP call, so invalid calls never touch the GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "nm_spmv.h"
#include "nm_kernels.h"

namespace {

thread_local char g_err[512] = "";

nm_status fail(nm_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

nm_status hip_fail(const char *what, hipError_t e) {
    return fail(NM_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu[kMaxDevices];
std::atomic<int> g_lds[kMaxDevices];

// Properties of the current device (cached).  Falls back to gfx950 figures when no
// device is visible, which only matters for the size queries.
nmk::DeviceInfo device_info() {
    nmk::DeviceInfo d;
    d.num_cu = 256;
    d.max_lds_per_block = 160 * 1024;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return d;
    }
    int cu = g_cu[dev].load(std::memory_order_relaxed);
    int lds = g_lds[dev].load(std::memory_order_relaxed);
    if (cu <= 0) {
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) {
            (void)hipGetLastError();
            cu = 256;
        }
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || lds <= 0) {
            (void)hipGetLastError();
            lds = 64 * 1024;
        }
        g_lds[dev].store(lds, std::memory_order_relaxed);
        g_cu[dev].store(cu, std::memory_order_relaxed);
    }
    d.num_cu = cu;
    d.max_lds_per_block = lds;
    return d;
}

nmk::MvPlan spmv_plan(int64_t R, int64_t K, int B, int fmt = nmk::kMetaBitmask) {
    return nmk::plan_spmv(R, K, B, device_info(), fmt);
}

// Plan of one launch over a validated set: the matrix-core tile kernel where it applies
// (bitmask, B >= 5, K a multiple of 1024), else the word-per-lane kernel.  At B = 3 or 4
// the tile kernel replaces the word-per-lane one only where the latter would cut K into
// slices for LDS on a matrix with rows for every CU (e.g. 4096 x 14336 at B = 4:
// 17.3 vs 19.7 us); elsewhere it is the slower of the two at these batch sizes.
nmk::MvPlan spmv_set_plan(const nmk::SpmvSet &set, int fmt, int64_t K, int64_t ldx, int B, int epi) {
    const int64_t R = set.row0[set.P];
    const nmk::MvPlan word = spmv_plan(R, K, B, fmt);
    if (nmk::spmv_tile_ok(set, K, ldx, B, fmt, epi)) {
        const int64_t cu = device_info().num_cu > 0 ? device_info().num_cu : 256;
        if (B >= nmk::kTileMinB || (word.splits > 1 && R >= 2 * cu))
            return nmk::plan_spmv_tile(set, K, B, device_info(), epi);
    }
    if (set.P == 1 && epi == nmk::kEpiNone && fmt == nmk::kMetaBitmask)
        return nmk::plan_spmv_one(word, R, K, B, device_info());
    return word;
}

nmk::MvPlan spmv_unstructured_plan(int64_t R, int64_t K, int B) {
    nmk::MvPlan p = nmk::plan_spmv_unstructured(R, K, B, device_info());
    return p;
}

nmk::MvPlan dense_plan(int64_t R, int64_t K, int B, int epi = nmk::kEpiNone) {
    return nmk::plan_dense(R, K, B, device_info(), epi);
}

constexpr int64_t kMaxDim = (int64_t)1 << 30;

nm_status check_mv_common(int64_t R, int64_t K, int B, int64_t ldx, int64_t ldy, const void *x, const void *y) {
    if (R < 1 || R > kMaxDim) return fail(NM_ERR_SHAPE, "R=%lld out of range [1, 2^30]", (long long)R);
    if (B < 1 || B > 8) return fail(NM_ERR_SHAPE, "B=%d out of range [1, 8]", B);
    if (ldx < K) return fail(NM_ERR_SHAPE, "ldx=%lld < K=%lld", (long long)ldx, (long long)K);
    if (ldy < R) return fail(NM_ERR_SHAPE, "ldy=%lld < R=%lld", (long long)ldy, (long long)R);
    if (ldx % 8) return fail(NM_ERR_ALIGN, "ldx=%lld is not a multiple of 8", (long long)ldx);
    if (!aligned(x, 16)) return fail(NM_ERR_ALIGN, "x is not 16-byte aligned");
    if (!aligned(y, 2)) return fail(NM_ERR_ALIGN, "y is not 2-byte aligned");
    return NM_OK;
}

}  // namespace

extern "C" {

const char *nm_status_str(int s) {
    switch (s) {
    case NM_OK: return "NM_OK";
    case NM_ERR_NULL: return "NM_ERR_NULL";
    case NM_ERR_SHAPE: return "NM_ERR_SHAPE";
    case NM_ERR_PATTERN: return "NM_ERR_PATTERN";
    case NM_ERR_ALIGN: return "NM_ERR_ALIGN";
    case NM_ERR_WORKSPACE: return "NM_ERR_WORKSPACE";
    case NM_ERR_HIP: return "NM_ERR_HIP";
    default: return "NM_ERR_UNKNOWN";
    }
}

const char *nm_last_error(void) { return g_err; }

int nm_version(void) { return 100; }

nm_status nm_col_norm(const nm_bf16 *X, int64_t T, int64_t K, int64_t ldx, float *col_norm, void *hip_stream) {
    try {
        g_err[0] = 0;
        if (!X || !col_norm) return fail(NM_ERR_NULL, "nm_col_norm: NULL pointer");
        if (T < 1 || T > kMaxDim || K < 1 || K > kMaxDim || ldx < K)
            return fail(NM_ERR_SHAPE, "nm_col_norm: bad sizes T=%lld K=%lld ldx=%lld", (long long)T, (long long)K,
                        (long long)ldx);
        if (!aligned(X, 2) || !aligned(col_norm, 4)) return fail(NM_ERR_ALIGN, "nm_col_norm: misaligned pointer");
        hipError_t e = nmk::launch_col_norm(X, T, K, ldx, col_norm, (hipStream_t)hip_stream);
        if (e != hipSuccess) return hip_fail("nm_col_norm launch", e);
        return NM_OK;
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_col_norm: internal error");
    }
}

nm_status nm_prune_pack(const nm_bf16 *W, int64_t ldw, int64_t R, int64_t K, const float *col_norm, int N, int M,
                        uint32_t *masks, nm_bf16 *values, void *hip_stream) {
    try {
        g_err[0] = 0;
        if (!W || !col_norm || !masks || !values) return fail(NM_ERR_NULL, "nm_prune_pack: NULL pointer");
        if (!(M == 4 || M == 8 || M == 16 || M == 32) || 2 * N != M)
            return fail(NM_ERR_PATTERN, "nm_prune_pack: %d:%d is not a 50%% pattern with M in {4,8,16,32}", N, M);
        if (R < 1 || R > kMaxDim || K < 32 || K > kMaxDim || K % 32 != 0 || ldw < K)
            return fail(NM_ERR_SHAPE, "nm_prune_pack: bad sizes R=%lld K=%lld ldw=%lld (K must be a multiple of 32)",
                        (long long)R, (long long)K, (long long)ldw);
        if (ldw % 8 || !aligned(W, 16) || !aligned(col_norm, 16) || !aligned(masks, 4) || !aligned(values, 16))
            return fail(NM_ERR_ALIGN, "nm_prune_pack: W/values/col_norm need 16-byte alignment, ldw a multiple of 8");
        hipError_t e = nmk::launch_prune_pack(W, ldw, R, K, col_norm, N, M, masks, values, (hipStream_t)hip_stream);
        if (e != hipSuccess) return hip_fail("nm_prune_pack launch", e);
        return NM_OK;
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_prune_pack: internal error");
    }
}

size_t nm_spmv_workspace_bytes(int64_t R, int64_t K, int B) {
    if (R < 1 || R > kMaxDim || K < 32 || K % 32 != 0 || K > kMaxDim || B < 1 || B > 8) return 0;
    return spmv_plan(R, K, B).ws_bytes;
}

// Shared body of nm_spmv / nm_spmv_multi once the matrices are validated into a set.
static nm_status spmv_run(const nmk::SpmvSet &set, int fmt, int64_t K, const nm_bf16 *x, int64_t ldx, int B,
                          void *workspace, size_t workspace_bytes, void *hip_stream, const char *who) {
    const nmk::MvPlan p = spmv_set_plan(set, fmt, K, ldx, B, nmk::kEpiNone);
    if (p.ws_bytes > 0) {
        if (!workspace || workspace_bytes < p.ws_bytes || !aligned(workspace, 4))
            return fail(NM_ERR_WORKSPACE, "%s: workspace of %zu bytes required, %zu given", who, p.ws_bytes,
                        workspace ? workspace_bytes : (size_t)0);
    }
    hipError_t e = p.tile ? nmk::launch_spmv_tile(p, set, K, x, ldx, B, nmk::kEpiNone, (hipStream_t)hip_stream)
                          : nmk::launch_spmv(p, set, fmt, K, x, ldx, B, (float *)workspace, (hipStream_t)hip_stream);
    if (e != hipSuccess) return hip_fail(who, e);
    return NM_OK;
}

// Shared body of nm_spmv / nm_spmv_meta (one matrix).
static nm_status spmv_one(const void *meta, int fmt, const nm_bf16 *values, int64_t R, int64_t K, const nm_bf16 *x,
                          int64_t ldx, int B, nm_bf16 *y, int64_t ldy, void *workspace, size_t workspace_bytes,
                          void *hip_stream, const char *who) {
    if (!meta || !values || !x || !y) return fail(NM_ERR_NULL, "%s: NULL pointer", who);
    if (fmt != NM_META_BITMASK && fmt != NM_META_U8_OFFSET && fmt != NM_META_I32_INDEX)
        return fail(NM_ERR_PATTERN, "%s: unknown metadata format %d", who, fmt);
    if (K < 32 || K > kMaxDim || K % 32 != 0)
        return fail(NM_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 32", who, (long long)K);
    nm_status st = check_mv_common(R, K, B, ldx, ldy, x, y);
    if (st != NM_OK) return st;
    if (!aligned(meta, fmt == NM_META_BITMASK ? 4 : 16) || !aligned(values, 16))
        return fail(NM_ERR_ALIGN, "%s: metadata needs 4-byte (masks) or 16-byte (index formats) and values 16-byte "
                                  "alignment", who);
    nmk::SpmvSet set;
    set.P = 1;
    set.row0[1] = (int)R;
    set.meta[0] = meta;
    set.values[0] = values;
    set.y[0] = y;
    set.ldy[0] = ldy;
    return spmv_run(set, fmt, K, x, ldx, B, workspace, workspace_bytes, hip_stream, who);
}

nm_status nm_spmv(const uint32_t *masks, const nm_bf16 *values, int64_t R, int64_t K, const nm_bf16 *x, int64_t ldx,
                  int B, nm_bf16 *y, int64_t ldy, void *workspace, size_t workspace_bytes, void *hip_stream) {
    try {
        g_err[0] = 0;
        return spmv_one(masks, NM_META_BITMASK, values, R, K, x, ldx, B, y, ldy, workspace, workspace_bytes,
                        hip_stream, "nm_spmv");
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_spmv: internal error");
    }
}

nm_status nm_spmv_noalloc(const uint32_t *masks, const nm_bf16 *values, int64_t R, int64_t K, const nm_bf16 *x,
                          int64_t ldx, int B, nm_bf16 *y, int64_t ldy, void *hip_stream) {
    try {
        g_err[0] = 0;
        const char *who = "nm_spmv_noalloc";
        if (!masks || !values || !x || !y) return fail(NM_ERR_NULL, "%s: NULL pointer", who);
        if (K < 32 || K > kMaxDim || K % 32 != 0)
            return fail(NM_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 32", who, (long long)K);
        nm_status st = check_mv_common(R, K, B, ldx, ldy, x, y);
        if (st != NM_OK) return st;
        if (!aligned(masks, 4) || !aligned(values, 16))
            return fail(NM_ERR_ALIGN, "%s: masks need 4-byte and values 16-byte alignment", who);
        nmk::SpmvSet set;
        set.P = 1;
        set.row0[1] = (int)R;
        set.meta[0] = masks;
        set.values[0] = values;
        set.y[0] = y;
        set.ldy[0] = ldy;
        const nmk::MvPlan p = spmv_set_plan(set, NM_META_BITMASK, K, ldx, B, nmk::kEpiNone);
        if (p.ws_bytes > nmk::kSpmvScratchBytes)
            return fail(NM_ERR_WORKSPACE, "%s: this shape needs %zu bytes of scratch, above the fixed %zu", who,
                        p.ws_bytes, nmk::kSpmvScratchBytes);
        void *scratch = nullptr;
        if (p.ws_bytes > 0) {
            hipError_t e = nmk::spmv_scratch(&scratch);
            if (e != hipSuccess) return hip_fail("nm_spmv_noalloc scratch lookup", e);
        }
        hipError_t e = p.tile ? nmk::launch_spmv_tile(p, set, K, x, ldx, B, nmk::kEpiNone, (hipStream_t)hip_stream)
                              : nmk::launch_spmv(p, set, NM_META_BITMASK, K, x, ldx, B, (float *)scratch,
                                                 (hipStream_t)hip_stream);
        if (e != hipSuccess) return hip_fail(who, e);
        return NM_OK;
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_spmv_noalloc: internal error");
    }
}

nm_status nm_spmv_meta(const void *meta, int format, const nm_bf16 *values, int64_t R, int64_t K, const nm_bf16 *x,
                       int64_t ldx, int B, nm_bf16 *y, int64_t ldy, void *workspace, size_t workspace_bytes,
                       void *hip_stream) {
    try {
        g_err[0] = 0;
        return spmv_one(meta, format, values, R, K, x, ldx, B, y, ldy, workspace, workspace_bytes, hip_stream,
                        "nm_spmv_meta");
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_spmv_meta: internal error");
    }
}

nm_status nm_meta_from_mask(const uint32_t *masks, int64_t R, int64_t K, int format, void *meta, void *hip_stream) {
    try {
        g_err[0] = 0;
        if (!masks || !meta) return fail(NM_ERR_NULL, "nm_meta_from_mask: NULL pointer");
        if (format != NM_META_U8_OFFSET && format != NM_META_I32_INDEX)
            return fail(NM_ERR_PATTERN, "nm_meta_from_mask: format %d is not an index format", format);
        if (R < 1 || R > kMaxDim || K < 32 || K > kMaxDim || K % 32 != 0)
            return fail(NM_ERR_SHAPE, "nm_meta_from_mask: bad sizes R=%lld K=%lld", (long long)R, (long long)K);
        if (!aligned(masks, 4) || !aligned(meta, 16))
            return fail(NM_ERR_ALIGN, "nm_meta_from_mask: masks need 4-byte and meta 16-byte alignment");
        hipError_t e = nmk::launch_meta_from_mask(masks, R, K, format, meta, (hipStream_t)hip_stream);
        if (e != hipSuccess) return hip_fail("nm_meta_from_mask launch", e);
        return NM_OK;
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_meta_from_mask: internal error");
    }
}

// Validates a host array of matrices sharing K into a set; 0 rows in total is an error.
static nm_status build_spmv_set(const nm_spmv_matrix *mats, int P, int64_t K, int B, nmk::SpmvSet &set,
                                const char *who) {
    if (!mats) return fail(NM_ERR_NULL, "%s: NULL matrix array", who);
    if (P < 1 || P > nmk::kMaxMats) return fail(NM_ERR_SHAPE, "%s: P=%d out of range [1, %d]", who, P, nmk::kMaxMats);
    if (K < 32 || K > kMaxDim || K % 32 != 0)
        return fail(NM_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 32", who, (long long)K);
    int64_t total = 0;
    set.P = P;
    for (int i = 0; i < P; ++i) {
        const nm_spmv_matrix &m = mats[i];
        if (!m.masks || !m.values || !m.y) return fail(NM_ERR_NULL, "%s: NULL pointer in matrix %d", who, i);
        if (m.R < 1 || m.R > kMaxDim) return fail(NM_ERR_SHAPE, "%s: matrix %d has R=%lld", who, i, (long long)m.R);
        if (m.ldy < m.R) return fail(NM_ERR_SHAPE, "%s: matrix %d has ldy < R", who, i);
        if (!aligned(m.masks, 4) || !aligned(m.values, 16) || !aligned(m.y, 2))
            return fail(NM_ERR_ALIGN, "%s: matrix %d misaligned (masks 4, values 16, y 2 bytes)", who, i);
        set.row0[i] = (int)total;
        set.meta[i] = m.masks;
        set.values[i] = m.values;
        set.y[i] = m.y;
        set.ldy[i] = m.ldy;
        total += m.R;
        if (total > kMaxDim) return fail(NM_ERR_SHAPE, "%s: more than 2^30 rows in total", who);
    }
    set.row0[P] = (int)total;
    (void)B;
    return NM_OK;
}

size_t nm_spmv_multi_workspace_bytes(const nm_spmv_matrix *mats, int P, int64_t K, int B) {
    if (!mats || P < 1 || P > nmk::kMaxMats || K < 32 || K % 32 != 0 || K > kMaxDim || B < 1 || B > 8) return 0;
    int64_t total = 0;
    for (int i = 0; i < P; ++i) {
        if (mats[i].R < 1) return 0;
        total += mats[i].R;
    }
    if (total > kMaxDim) return 0;
    return spmv_plan(total, K, B).ws_bytes;
}

nm_status nm_spmv_multi(const nm_spmv_matrix *mats, int P, int64_t K, const nm_bf16 *x, int64_t ldx, int B,
                        void *workspace, size_t workspace_bytes, void *hip_stream) {
    try {
        g_err[0] = 0;
        if (!x) return fail(NM_ERR_NULL, "nm_spmv_multi: NULL x");
        nmk::SpmvSet set;
        nm_status st = build_spmv_set(mats, P, K, B, set, "nm_spmv_multi");
        if (st != NM_OK) return st;
        if (B < 1 || B > 8) return fail(NM_ERR_SHAPE, "nm_spmv_multi: B=%d out of range [1, 8]", B);
        if (ldx < K) return fail(NM_ERR_SHAPE, "nm_spmv_multi: ldx < K");
        if (ldx % 8 || !aligned(x, 16)) return fail(NM_ERR_ALIGN, "nm_spmv_multi: x needs 16-byte alignment, ldx % 8 == 0");
        return spmv_run(set, NM_META_BITMASK, K, x, ldx, B, workspace, workspace_bytes, hip_stream, "nm_spmv_multi");
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_spmv_multi: internal error");
    }
}

size_t nm_spmv_swiglu_workspace_bytes(int64_t R, int64_t K, int B) {
    if (R < 1 || R > kMaxDim / 2 || K < 32 || K % 32 != 0 || K > kMaxDim || B < 1 || B > 8) return 0;
    return spmv_plan(2 * R, K, B).ws_bytes;
}

nm_status nm_spmv_swiglu(const uint32_t *gate_masks, const nm_bf16 *gate_values, const uint32_t *up_masks,
                         const nm_bf16 *up_values, int64_t R, int64_t K, const nm_bf16 *x, int64_t ldx, int B,
                         nm_bf16 *h, int64_t ldh, void *workspace, size_t workspace_bytes, void *hip_stream) {
    try {
        g_err[0] = 0;
        const char *who = "nm_spmv_swiglu";
        if (!gate_masks || !gate_values || !up_masks || !up_values || !x || !h)
            return fail(NM_ERR_NULL, "%s: NULL pointer", who);
        if (K < 32 || K > kMaxDim || K % 32 != 0)
            return fail(NM_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 32", who, (long long)K);
        if (R > kMaxDim / 2) return fail(NM_ERR_SHAPE, "%s: R=%lld above 2^29", who, (long long)R);
        nm_status st = check_mv_common(R, K, B, ldx, ldh, x, h);
        if (st != NM_OK) return st;
        if (!aligned(gate_masks, 4) || !aligned(up_masks, 4) || !aligned(gate_values, 16) || !aligned(up_values, 16))
            return fail(NM_ERR_ALIGN, "%s: masks need 4-byte and values 16-byte alignment", who);
        nmk::SpmvSet set;
        set.P = 2;
        set.row0[1] = (int)R;
        set.row0[2] = (int)(2 * R);
        set.meta[0] = gate_masks;
        set.values[0] = gate_values;
        set.meta[1] = up_masks;
        set.values[1] = up_values;
        set.y[0] = h;
        set.ldy[0] = ldh;
        set.y[1] = h;  // unused: the epilogue writes matrix 0's output only
        set.ldy[1] = ldh;
        const nmk::MvPlan p = spmv_set_plan(set, NM_META_BITMASK, K, ldx, B, nmk::kEpiSwiGLU);
        if (p.ws_bytes > 0) {
            if (!workspace || workspace_bytes < p.ws_bytes || !aligned(workspace, 4))
                return fail(NM_ERR_WORKSPACE, "%s: workspace of %zu bytes required, %zu given", who, p.ws_bytes,
                            workspace ? workspace_bytes : (size_t)0);
        }
        hipError_t e = p.tile
                           ? nmk::launch_spmv_tile(p, set, K, x, ldx, B, nmk::kEpiSwiGLU, (hipStream_t)hip_stream)
                           : nmk::launch_spmv_swiglu(p, set, K, x, ldx, B, (float *)workspace,
                                                     (hipStream_t)hip_stream);
        if (e != hipSuccess) return hip_fail(who, e);
        return NM_OK;
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_spmv_swiglu: internal error");
    }
}

static void fill_plan(const nmk::MvPlan &p, nm_launch_plan *out) {
    out->kernel = p.tile                             ? NM_KERNEL_TILE
                  : p.walk == nmk::kWalkHalf   ? NM_KERNEL_WORD_HALF_ROWS
                  : p.walk == nmk::kWalkStrips ? NM_KERNEL_WORD_STRIPS
                                               : NM_KERNEL_WORD;
    out->threads = p.threads;
    out->grid_x = p.grid_x;
    out->splits = p.splits;
    out->tiles_per_step = p.tile ? p.unroll : 0;
    out->x_steps_in_registers = p.tile ? p.xreg : 0;
    out->rows_per_group = p.walk == nmk::kWalkStrips ? p.rows_per_group : 0;
    out->lds_bytes = p.tile ? 0 : p.lds_bytes;
    out->workspace_bytes = p.ws_bytes;
}

nm_status nm_spmv_plan(int64_t R, int64_t K, int B, int epilogue, nm_launch_plan *plan) {
    try {
        g_err[0] = 0;
        if (!plan) return fail(NM_ERR_NULL, "nm_spmv_plan: NULL plan");
        if (epilogue != NM_EPI_NONE && epilogue != NM_EPI_SWIGLU)
            return fail(NM_ERR_PATTERN, "nm_spmv_plan: unknown epilogue %d", epilogue);
        const int64_t rmax = epilogue == NM_EPI_SWIGLU ? kMaxDim / 2 : kMaxDim;
        if (R < 1 || R > rmax || K < 32 || K > kMaxDim || K % 32 != 0 || B < 1 || B > 8)
            return fail(NM_ERR_SHAPE, "nm_spmv_plan: bad sizes R=%lld K=%lld B=%d", (long long)R, (long long)K, B);
        nmk::SpmvSet set;
        if (epilogue == NM_EPI_SWIGLU) {
            set.P = 2;
            set.row0[1] = (int)R;
            set.row0[2] = (int)(2 * R);
        } else {
            set.P = 1;
            set.row0[1] = (int)R;
        }
        const int epi = epilogue == NM_EPI_SWIGLU ? nmk::kEpiSwiGLU : nmk::kEpiNone;
        fill_plan(spmv_set_plan(set, NM_META_BITMASK, K, K, B, epi), plan);
        return NM_OK;
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_spmv_plan: internal error");
    }
}

nm_status nm_spmv_multi_plan(const int64_t *rows, int P, int64_t K, int B, nm_launch_plan *plan) {
    try {
        g_err[0] = 0;
        if (!plan || !rows) return fail(NM_ERR_NULL, "nm_spmv_multi_plan: NULL pointer");
        if (P < 1 || P > nmk::kMaxMats || K < 32 || K > kMaxDim || K % 32 != 0 || B < 1 || B > 8)
            return fail(NM_ERR_SHAPE, "nm_spmv_multi_plan: bad sizes P=%d K=%lld B=%d", P, (long long)K, B);
        nmk::SpmvSet set;
        int64_t total = 0;
        set.P = P;
        for (int i = 0; i < P; ++i) {
            if (rows[i] < 1 || rows[i] > kMaxDim)
                return fail(NM_ERR_SHAPE, "nm_spmv_multi_plan: matrix %d has R=%lld", i, (long long)rows[i]);
            set.row0[i] = (int)total;
            total += rows[i];
            if (total > kMaxDim) return fail(NM_ERR_SHAPE, "nm_spmv_multi_plan: more than 2^30 rows in total");
        }
        set.row0[P] = (int)total;
        fill_plan(spmv_set_plan(set, NM_META_BITMASK, K, K, B, nmk::kEpiNone), plan);
        return NM_OK;
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_spmv_multi_plan: internal error");
    }
}

nm_status nm_prune_pack_unstructured(const nm_bf16 *W, int64_t ldw, int64_t R, int64_t K, const float *col_norm,
                                     uint32_t *masks, nm_bf16 *values, void *hip_stream) {
    try {
        g_err[0] = 0;
        if (!W || !col_norm || !masks || !values) return fail(NM_ERR_NULL, "nm_prune_pack_unstructured: NULL pointer");
        if (R < 1 || R > kMaxDim || K < 32 || K > kMaxDim || K % 32 != 0 || ldw < K)
            return fail(NM_ERR_SHAPE, "nm_prune_pack_unstructured: bad sizes R=%lld K=%lld ldw=%lld", (long long)R,
                        (long long)K, (long long)ldw);
        if (ldw % 8 || !aligned(W, 16) || !aligned(col_norm, 16) || !aligned(masks, 4) || !aligned(values, 2))
            return fail(NM_ERR_ALIGN, "nm_prune_pack_unstructured: W/col_norm need 16-byte alignment, ldw % 8 == 0");
        hipError_t e = nmk::launch_prune_pack_unstructured(W, ldw, R, K, col_norm, masks, values,
                                                           (hipStream_t)hip_stream);
        if (e != hipSuccess) return hip_fail("nm_prune_pack_unstructured launch", e);
        return NM_OK;
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_prune_pack_unstructured: internal error");
    }
}

size_t nm_spmv_unstructured_workspace_bytes(int64_t R, int64_t K, int B) {
    if (R < 1 || R > kMaxDim || K < 32 || K % 32 != 0 || K > kMaxDim || B < 1 || B > 8) return 0;
    return spmv_unstructured_plan(R, K, B).ws_bytes;
}

nm_status nm_spmv_unstructured(const uint32_t *masks, const nm_bf16 *values, int64_t R, int64_t K, const nm_bf16 *x,
                               int64_t ldx, int B, nm_bf16 *y, int64_t ldy, void *workspace, size_t workspace_bytes,
                               void *hip_stream) {
    try {
        g_err[0] = 0;
        const char *who = "nm_spmv_unstructured";
        if (!masks || !values || !x || !y) return fail(NM_ERR_NULL, "%s: NULL pointer", who);
        if (K < 32 || K > kMaxDim || K % 32 != 0)
            return fail(NM_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 32", who, (long long)K);
        nm_status st = check_mv_common(R, K, B, ldx, ldy, x, y);
        if (st != NM_OK) return st;
        if (!aligned(masks, 4) || !aligned(values, 16))
            return fail(NM_ERR_ALIGN, "%s: masks need 4-byte and values 16-byte alignment", who);
        const nmk::MvPlan p = spmv_unstructured_plan(R, K, B);
        if (p.ws_bytes > 0) {
            if (!workspace || workspace_bytes < p.ws_bytes || !aligned(workspace, 4))
                return fail(NM_ERR_WORKSPACE, "%s: workspace of %zu bytes required, %zu given", who, p.ws_bytes,
                            workspace ? workspace_bytes : (size_t)0);
        }
        hipError_t e = nmk::launch_spmv_unstructured(p, masks, values, R, K, x, ldx, B, y, ldy, (float *)workspace,
                                                     (hipStream_t)hip_stream);
        if (e != hipSuccess) return hip_fail(who, e);
        return NM_OK;
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_spmv_unstructured: internal error");
    }
}

nm_status nm_unpack_unstructured(const uint32_t *masks, const nm_bf16 *values, int64_t R, int64_t K, nm_bf16 *W_out,
                                 int64_t ldw, void *hip_stream) {
    try {
        g_err[0] = 0;
        if (!masks || !values || !W_out) return fail(NM_ERR_NULL, "nm_unpack_unstructured: NULL pointer");
        if (R < 1 || R > kMaxDim || K < 32 || K > kMaxDim || K % 32 != 0 || ldw < K)
            return fail(NM_ERR_SHAPE, "nm_unpack_unstructured: bad sizes R=%lld K=%lld ldw=%lld", (long long)R,
                        (long long)K, (long long)ldw);
        if (ldw % 8 || !aligned(W_out, 16) || !aligned(values, 2) || !aligned(masks, 4))
            return fail(NM_ERR_ALIGN, "nm_unpack_unstructured: W_out needs 16-byte alignment, ldw % 8 == 0");
        hipError_t e = nmk::launch_unpack_unstructured(masks, values, R, K, W_out, ldw, (hipStream_t)hip_stream);
        if (e != hipSuccess) return hip_fail("nm_unpack_unstructured launch", e);
        return NM_OK;
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_unpack_unstructured: internal error");
    }
}

// ---------------------------------------------------------------- OBS / SparseGPT solver
constexpr int64_t kMaxSolverK = 65536;

nm_status nm_hessian(const nm_bf16 *X, int64_t T, int64_t K, int64_t ldx, double *H, int64_t ldh, void *hip_stream) {
    try {
        g_err[0] = 0;
        if (!X || !H) return fail(NM_ERR_NULL, "nm_hessian: NULL pointer");
        if (T < 1 || T > kMaxDim || K < 1 || K > kMaxSolverK || ldx < K || ldh < K)
            return fail(NM_ERR_SHAPE, "nm_hessian: bad sizes T=%lld K=%lld ldx=%lld ldh=%lld", (long long)T,
                        (long long)K, (long long)ldx, (long long)ldh);
        if (!aligned(X, 2) || !aligned(H, 8)) return fail(NM_ERR_ALIGN, "nm_hessian: misaligned pointer");
        hipError_t e = nmk::launch_hessian(X, T, K, ldx, H, ldh, (hipStream_t)hip_stream);
        if (e != hipSuccess) return hip_fail("nm_hessian launch", e);
        return NM_OK;
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_hessian: internal error");
    }
}

size_t nm_obs_inverse_factor_workspace_bytes(int64_t K) {
    if (K < 32 || K % 32 != 0 || K > kMaxSolverK) return 0;
    return nmk::sparsegpt_factor_workspace(K);
}

static nm_status check_solver_h(const double *H, int64_t ldh, int64_t K, double damp, const char *who) {
    if (!H) return fail(NM_ERR_NULL, "%s: NULL H", who);
    if (K < 32 || K % 32 != 0 || K > kMaxSolverK || ldh < K)
        return fail(NM_ERR_SHAPE, "%s: K=%lld must be a multiple of 32 in [32, 65536], ldh >= K", who, (long long)K);
    if (!(damp >= 0.0) || damp > 1e30) return fail(NM_ERR_SHAPE, "%s: damp must be finite and >= 0", who);
    if (!aligned(H, 8)) return fail(NM_ERR_ALIGN, "%s: H needs 8-byte alignment", who);
    return NM_OK;
}

nm_status nm_obs_inverse_factor(const double *H, int64_t ldh, int64_t K, double damp, double *U, int64_t ldu,
                                void *workspace, size_t workspace_bytes, void *hip_stream) {
    try {
        g_err[0] = 0;
        const char *who = "nm_obs_inverse_factor";
        nm_status st = check_solver_h(H, ldh, K, damp, who);
        if (st != NM_OK) return st;
        if (!U) return fail(NM_ERR_NULL, "%s: NULL U", who);
        if (ldu < K) return fail(NM_ERR_SHAPE, "%s: ldu < K", who);
        if (!aligned(U, 8)) return fail(NM_ERR_ALIGN, "%s: U needs 8-byte alignment", who);
        const size_t need = nmk::sparsegpt_factor_workspace(K);
        if (!workspace || workspace_bytes < need || !aligned(workspace, 8))
            return fail(NM_ERR_WORKSPACE, "%s: workspace of %zu bytes required, %zu given", who, need,
                        workspace ? workspace_bytes : (size_t)0);
        hipError_t e = nmk::launch_inverse_factor(H, ldh, K, damp, U, ldu, workspace, (hipStream_t)hip_stream);
        if (e != hipSuccess) return hip_fail(who, e);
        return NM_OK;
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_obs_inverse_factor: internal error");
    }
}

size_t nm_sparsegpt_workspace_bytes(int64_t R, int64_t K) {
    if (R < 1 || R > kMaxDim || K < 32 || K % 32 != 0 || K > kMaxSolverK) return 0;
    return nmk::sparsegpt_workspace(R, K);
}

nm_status nm_sparsegpt_prune_pack(const nm_bf16 *W, int64_t ldw, int64_t R, int64_t K, const double *H, int64_t ldh,
                                  int N, int M, double damp, uint32_t *masks, nm_bf16 *values, void *workspace,
                                  size_t workspace_bytes, void *hip_stream) {
    try {
        g_err[0] = 0;
        const char *who = "nm_sparsegpt_prune_pack";
        if (!W || !masks || !values) return fail(NM_ERR_NULL, "%s: NULL pointer", who);
        if (!(M == 4 || M == 8 || M == 16 || M == 32) || 2 * N != M)
            return fail(NM_ERR_PATTERN, "%s: %d:%d is not a 50%% pattern with M in {4,8,16,32}", who, N, M);
        nm_status st = check_solver_h(H, ldh, K, damp, who);
        if (st != NM_OK) return st;
        if (R < 1 || R > kMaxDim || ldw < K) return fail(NM_ERR_SHAPE, "%s: bad sizes R=%lld ldw=%lld", who,
                                                         (long long)R, (long long)ldw);
        if (!aligned(W, 2) || !aligned(masks, 4) || !aligned(values, 16))
            return fail(NM_ERR_ALIGN, "%s: W 2-byte, masks 4-byte and values 16-byte alignment required", who);
        const size_t need = nmk::sparsegpt_workspace(R, K);
        if (!workspace || workspace_bytes < need || !aligned(workspace, 8))
            return fail(NM_ERR_WORKSPACE, "%s: workspace of %zu bytes required, %zu given", who, need,
                        workspace ? workspace_bytes : (size_t)0);
        hipError_t e = nmk::launch_sparsegpt(W, ldw, R, K, H, ldh, N, M, damp, masks, values, workspace,
                                             (hipStream_t)hip_stream);
        if (e != hipSuccess) return hip_fail(who, e);
        return NM_OK;
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_sparsegpt_prune_pack: internal error");
    }
}

size_t dense_gemv_workspace_bytes(int64_t R, int64_t K, int B) {
    if (R < 1 || R > kMaxDim || K < 8 || K % 8 != 0 || K > kMaxDim || B < 1 || B > 8) return 0;
    return dense_plan(R, K, B).ws_bytes;
}

static nm_status dense_run(const nmk::DenseSet &set, int64_t K, const nm_bf16 *x, int64_t ldx, int B,
                           void *workspace, size_t workspace_bytes, void *hip_stream, const char *who) {
    const int64_t R = set.row0[set.P];
    const nmk::MvPlan p = dense_plan(R, K, B);
    if (p.ws_bytes > 0) {
        if (!workspace || workspace_bytes < p.ws_bytes || !aligned(workspace, 4))
            return fail(NM_ERR_WORKSPACE, "%s: workspace of %zu bytes required, %zu given", who, p.ws_bytes,
                        workspace ? workspace_bytes : (size_t)0);
    }
    hipError_t e = nmk::launch_dense(p, set, K, x, ldx, B, (float *)workspace, (hipStream_t)hip_stream);
    if (e != hipSuccess) return hip_fail(who, e);
    return NM_OK;
}

nm_status dense_gemv(const nm_bf16 *W, int64_t ldw, int64_t R, int64_t K, const nm_bf16 *x, int64_t ldx, int B,
                     nm_bf16 *y, int64_t ldy, void *workspace, size_t workspace_bytes, void *hip_stream) {
    try {
        g_err[0] = 0;
        if (!W || !x || !y) return fail(NM_ERR_NULL, "dense_gemv: NULL pointer");
        if (K < 8 || K > kMaxDim || K % 8 != 0 || ldw < K)
            return fail(NM_ERR_SHAPE, "dense_gemv: bad sizes K=%lld ldw=%lld (K must be a multiple of 8)",
                        (long long)K, (long long)ldw);
        nm_status st = check_mv_common(R, K, B, ldx, ldy, x, y);
        if (st != NM_OK) return st;
        if (ldw % 8 || !aligned(W, 16))
            return fail(NM_ERR_ALIGN, "dense_gemv: W needs 16-byte alignment and ldw a multiple of 8");
        nmk::DenseSet set;
        set.P = 1;
        set.row0[1] = (int)R;
        set.W[0] = W;
        set.ldw[0] = ldw;
        set.y[0] = y;
        set.ldy[0] = ldy;
        return dense_run(set, K, x, ldx, B, workspace, workspace_bytes, hip_stream, "dense_gemv");
    } catch (...) {
        return fail(NM_ERR_HIP, "dense_gemv: internal error");
    }
}

size_t dense_gemv_swiglu_workspace_bytes(int64_t R, int64_t K, int B) {
    if (R < 1 || R > kMaxDim / 2 || K < 8 || K % 8 != 0 || K > kMaxDim || B < 1 || B > 8) return 0;
    return dense_plan(2 * R, K, B, nmk::kEpiSwiGLU).ws_bytes;
}

nm_status dense_gemv_swiglu(const nm_bf16 *W_gate, const nm_bf16 *W_up, int64_t ldw, int64_t R, int64_t K,
                            const nm_bf16 *x, int64_t ldx, int B, nm_bf16 *h, int64_t ldh, void *workspace,
                            size_t workspace_bytes, void *hip_stream) {
    try {
        g_err[0] = 0;
        const char *who = "dense_gemv_swiglu";
        if (!W_gate || !W_up || !x || !h) return fail(NM_ERR_NULL, "%s: NULL pointer", who);
        if (K < 8 || K > kMaxDim || K % 8 != 0 || ldw < K)
            return fail(NM_ERR_SHAPE, "%s: bad sizes K=%lld ldw=%lld", who, (long long)K, (long long)ldw);
        if (R > kMaxDim / 2) return fail(NM_ERR_SHAPE, "%s: R=%lld above 2^29", who, (long long)R);
        nm_status st = check_mv_common(R, K, B, ldx, ldh, x, h);
        if (st != NM_OK) return st;
        if (ldw % 8 || !aligned(W_gate, 16) || !aligned(W_up, 16))
            return fail(NM_ERR_ALIGN, "%s: W needs 16-byte alignment and ldw a multiple of 8", who);
        nmk::DenseSet set;
        set.P = 2;
        set.row0[1] = (int)R;
        set.row0[2] = (int)(2 * R);
        set.W[0] = W_gate;
        set.W[1] = W_up;
        set.ldw[0] = set.ldw[1] = ldw;
        set.y[0] = set.y[1] = h;
        set.ldy[0] = set.ldy[1] = ldh;
        const nmk::MvPlan p = dense_plan(2 * R, K, B, nmk::kEpiSwiGLU);
        if (p.ws_bytes > 0) {
            if (!workspace || workspace_bytes < p.ws_bytes || !aligned(workspace, 4))
                return fail(NM_ERR_WORKSPACE, "%s: workspace of %zu bytes required, %zu given", who, p.ws_bytes,
                            workspace ? workspace_bytes : (size_t)0);
        }
        hipError_t e = nmk::launch_dense_swiglu(p, set, K, x, ldx, B, (float *)workspace, (hipStream_t)hip_stream);
        if (e != hipSuccess) return hip_fail(who, e);
        return NM_OK;
    } catch (...) {
        return fail(NM_ERR_HIP, "dense_gemv_swiglu: internal error");
    }
}

size_t dense_gemv_multi_workspace_bytes(const dense_matrix *mats, int P, int64_t K, int B) {
    if (!mats || P < 1 || P > nmk::kMaxMats || K < 8 || K % 8 != 0 || K > kMaxDim || B < 1 || B > 8) return 0;
    int64_t total = 0;
    for (int i = 0; i < P; ++i) {
        if (mats[i].R < 1) return 0;
        total += mats[i].R;
    }
    if (total > kMaxDim) return 0;
    return dense_plan(total, K, B).ws_bytes;
}

nm_status dense_gemv_multi(const dense_matrix *mats, int P, int64_t K, const nm_bf16 *x, int64_t ldx, int B,
                           void *workspace, size_t workspace_bytes, void *hip_stream) {
    try {
        g_err[0] = 0;
        if (!mats || !x) return fail(NM_ERR_NULL, "dense_gemv_multi: NULL pointer");
        if (P < 1 || P > nmk::kMaxMats) return fail(NM_ERR_SHAPE, "dense_gemv_multi: P=%d out of range", P);
        if (K < 8 || K > kMaxDim || K % 8 != 0) return fail(NM_ERR_SHAPE, "dense_gemv_multi: K=%lld", (long long)K);
        if (B < 1 || B > 8) return fail(NM_ERR_SHAPE, "dense_gemv_multi: B=%d out of range [1, 8]", B);
        if (ldx < K) return fail(NM_ERR_SHAPE, "dense_gemv_multi: ldx < K");
        if (ldx % 8 || !aligned(x, 16)) return fail(NM_ERR_ALIGN, "dense_gemv_multi: x alignment");
        nmk::DenseSet set;
        int64_t total = 0;
        set.P = P;
        for (int i = 0; i < P; ++i) {
            const dense_matrix &m = mats[i];
            if (!m.W || !m.y) return fail(NM_ERR_NULL, "dense_gemv_multi: NULL pointer in matrix %d", i);
            if (m.R < 1 || m.R > kMaxDim || m.ldw < K || m.ldy < m.R)
                return fail(NM_ERR_SHAPE, "dense_gemv_multi: bad sizes in matrix %d", i);
            if (m.ldw % 8 || !aligned(m.W, 16) || !aligned(m.y, 2))
                return fail(NM_ERR_ALIGN, "dense_gemv_multi: matrix %d misaligned", i);
            set.row0[i] = (int)total;
            set.W[i] = m.W;
            set.ldw[i] = m.ldw;
            set.y[i] = m.y;
            set.ldy[i] = m.ldy;
            total += m.R;
            if (total > kMaxDim) return fail(NM_ERR_SHAPE, "dense_gemv_multi: more than 2^30 rows");
        }
        set.row0[P] = (int)total;
        return dense_run(set, K, x, ldx, B, workspace, workspace_bytes, hip_stream, "dense_gemv_multi");
    } catch (...) {
        return fail(NM_ERR_HIP, "dense_gemv_multi: internal error");
    }
}

nm_status nm_unpack(const uint32_t *masks, const nm_bf16 *values, int64_t R, int64_t K, nm_bf16 *W_out, int64_t ldw,
                    void *hip_stream) {
    try {
        g_err[0] = 0;
        if (!masks || !values || !W_out) return fail(NM_ERR_NULL, "nm_unpack: NULL pointer");
        if (R < 1 || R > kMaxDim || K < 32 || K > kMaxDim || K % 32 != 0 || ldw < K)
            return fail(NM_ERR_SHAPE, "nm_unpack: bad sizes R=%lld K=%lld ldw=%lld", (long long)R, (long long)K,
                        (long long)ldw);
        if (ldw % 8 || !aligned(W_out, 16) || !aligned(values, 16) || !aligned(masks, 4))
            return fail(NM_ERR_ALIGN, "nm_unpack: W_out/values need 16-byte alignment, ldw a multiple of 8");
        hipError_t e = nmk::launch_unpack(masks, values, R, K, W_out, ldw, (hipStream_t)hip_stream);
        if (e != hipSuccess) return hip_fail("nm_unpack launch", e);
        return NM_OK;
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_unpack: internal error");
    }
}

size_t nm_stream_read_sink_words(size_t bytes) { return nmk::stream_read_waves(bytes); }

nm_status nm_stream_read(const void *buf, size_t bytes, uint32_t *sink, size_t sink_words, void *hip_stream) {
    try {
        g_err[0] = 0;
        if (!buf || !sink) return fail(NM_ERR_NULL, "nm_stream_read: NULL pointer");
        if (bytes < 16 || bytes % 16 != 0 || bytes > ((size_t)1 << 31))
            return fail(NM_ERR_SHAPE, "nm_stream_read: bytes=%zu must be a multiple of 16 in [16, 2^31]", bytes);
        if (!aligned(buf, 16) || !aligned(sink, 4))
            return fail(NM_ERR_ALIGN, "nm_stream_read: buf needs 16-byte alignment");
        const size_t need = nmk::stream_read_waves(bytes);
        if (sink_words < need)
            return fail(NM_ERR_WORKSPACE, "nm_stream_read: sink of %zu words required, %zu given", need, sink_words);
        hipError_t e = nmk::launch_stream_read(buf, bytes, sink, (hipStream_t)hip_stream);
        if (e != hipSuccess) return hip_fail("nm_stream_read launch", e);
        return NM_OK;
    } catch (...) {
        return fail(NM_ERR_HIP, "nm_stream_read: internal error");
    }
}

}  // extern "C"
