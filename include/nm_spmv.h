/*
 * nm_spmv.h -- C ABI of the N:M bitmask sparse decode library for AMD MI355X (gfx950).
 *
 * The library computes, on one GPU, the decode-time hot path of N:M-pruned linear
 * layers described on these pages (cited by title and section):
 *
 *   [SD-en]    "SparseDecoding: Decoding-Aware Pruning for Accurate and Efficient LLM
 *              Inference" (ai.info AI summary): Key Contributions 2; Main Findings
 *              (metadata reduction, identical traffic across patterns); Methodology in
 *              Plain English, Steps 2 and 3.
 *   [SD-cn]    "SparseDecoding:解码感知的准确高效大模型剪枝框架" (paper.rainbus.top):
 *              前置知识 (Prefill 与 Decoding; N:M 半结构化稀疏; SpMM 与 SpMV);
 *              核心方法 (核心创新二); 方法步骤详情 (第三步, 第四步).
 *   [SD-repro] "SparseDecoding：只用解码激活校准的稀疏推理" (daiwk.github.io):
 *              核心公式; 背景与主要改动.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers owned by the caller unless stated otherwise.  The
 *    library never allocates or frees device memory and keeps no per-call state.
 *  - bf16 tensors are passed as raw 16-bit patterns (nm_bf16).
 *  - Matrices are row-major; ld* arguments are row strides in ELEMENTS.
 *  - Every call is asynchronous on `hip_stream` (a hipStream_t; NULL = the default
 *    stream) and returns once the work is enqueued.  Argument errors are reported
 *    synchronously, before any HIP call is made; a fault inside a kernel surfaces at
 *    the caller's next synchronisation, as usual in HIP.
 *  - Inputs must be finite.  Behaviour on NaN/Inf inputs is unspecified.
 *  - Sizes (R, K, T) are limited to 2^30.
 *  - Alignment: the base pointers of W, values, x and col_norm (pack input) must be
 *    16-byte aligned and ldw, ldx must be multiples of 8 elements, else NM_ERR_ALIGN.
 *    masks and workspace must be 4-byte aligned, y 2-byte aligned (ldy is free);
 *    index metadata (nm_spmv_meta) 16-byte aligned.
 *  - Entry points are thread-safe and reentrant.  nm_last_error() returns a
 *    thread-local description of the last failure on the calling thread.
 *  - No C++ exception crosses this boundary.
 */
#ifndef NM_SPMV_H
#define NM_SPMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t nm_bf16; /* raw bfloat16 bits */

typedef enum {
    NM_OK = 0,
    NM_ERR_NULL = 1,      /* a required pointer is NULL                              */
    NM_ERR_SHAPE = 2,     /* sizes out of range / inconsistent (e.g. K % 32 != 0)    */
    NM_ERR_PATTERN = 3,   /* N:M not one of 2:4, 4:8, 8:16, 16:32                    */
    NM_ERR_ALIGN = 4,     /* pointer or leading dimension misaligned                 */
    NM_ERR_WORKSPACE = 5, /* workspace NULL or smaller than *_workspace_bytes()      */
    NM_ERR_HIP = 6        /* a HIP runtime call failed (message in nm_last_error)    */
} nm_status;

/* Static string naming a status code. */
const char *nm_status_str(int status);

/* Thread-local text of the last failure on this thread ("" if none). */
const char *nm_last_error(void);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int nm_version(void);

/*
 * nm_col_norm -- Wanda's per-input-channel activation norm [SD-repro, 核心公式]:
 *     col_norm[j] = sqrt( sum_{t < T} X[t][j]^2 ).
 * X: bf16 [T][ldx] calibration activations (one row per calibration token).
 * col_norm: fp32 [K] output.
 * The sum runs in fp64 in token order, the square root is the correctly rounded fp64
 * one, and the result is rounded once (to nearest even) to fp32.  The result is
 * therefore fully determined by X (bit-reproducible).
 * Requires 1 <= T <= 2^30, 1 <= K <= 2^30, ldx >= K.
 */
nm_status nm_col_norm(const nm_bf16 *X, int64_t T, int64_t K, int64_t ldx, float *col_norm,
                      void *hip_stream);

/*
 * nm_prune_pack -- Wanda-style N:M selection and bitmask packing.
 * Score [SD-repro, 核心公式]: s_ij = |W_ij| * col_norm[j], evaluated exactly (fp64
 * product of an 8-bit and a 24-bit significand).  In every group of M consecutive
 * input columns of a row the N highest scores are kept [SD-cn, 前置知识 N:M]; equal
 * scores keep the lower column.  Only 50% patterns are accepted: (N, M) in
 * {(2,4), (4,8), (8,16), (16,32)}, so that every aligned 32-column word holds exactly
 * 16 kept weights [SD-en, Methodology Step 3].
 *
 * Outputs (canonical packed layout [SD-en, Methodology Step 2]):
 *   masks  uint32 [R][K/32]: bit b of word w is set iff column 32w+b is kept.
 *   values bf16   [R][K/2] : values[i][16w+t] is the raw W pattern of the t-th kept
 *                            column of word w, in increasing column order (the order
 *                            a lowest-set-bit-first scan visits them).  A kept weight
 *                            whose value is zero still sets its bit.
 * W: bf16 [R][ldw], col_norm: fp32 [K] (non-negative, e.g. from nm_col_norm).
 * Requires R >= 1, K >= 32, K % 32 == 0, ldw >= K.
 */
nm_status nm_prune_pack(const nm_bf16 *W, int64_t ldw, int64_t R, int64_t K, const float *col_norm,
                        int N, int M, uint32_t *masks, nm_bf16 *values, void *hip_stream);

/*
 * nm_spmv -- batch-one (B <= 8) N:M sparse matrix-vector product of a packed matrix
 * [SD-en, Methodology Steps 2-3; SD-cn, 方法步骤详情 第四步]:
 *     y[b][i] = sum_j Wsparse[i][j] * x[b][j],   0 <= b < B, 0 <= i < R.
 * Each mask word is walked with a fixed 16-step loop (find lowest set bit -> column,
 * clear it), pairing the t-th set bit with values[16w+t].  The kernel does not depend
 * on M: every 50% pattern has 16 set bits per word.  Products and sums are fp32; y is
 * rounded to nearest even bf16.  For 5 <= B <= 8 and K a multiple of 1024 (and for
 * B = 3 or 4 with such a K above 10240 on at least two rows per compute unit) the walk
 * writes each kept value into a dense 16-row tile in LDS and the tile is multiplied by
 * the B inputs on the matrix cores (bf16 products, fp32 sums); that path uses no
 * workspace (the size query covers both paths).
 *
 * masks/values: canonical layout as produced by nm_prune_pack (rows contiguous).
 * x: bf16 [B][ldx]; y: bf16 [B][ldy] (ldy >= R).
 * workspace: device scratch of at least nm_spmv_workspace_bytes(R, K, B) bytes (may
 * be NULL when that size is 0).  It holds fp32 partial sums of split rows; the
 * second pass adds them in a fixed order, so results are bit-reproducible run to run.
 * Requires R >= 1, K >= 32, K % 32 == 0, 1 <= B <= 8, ldx >= K, ldy >= R, and every
 * mask word to hold exactly 16 set bits (not re-checked on the device).
 */
size_t nm_spmv_workspace_bytes(int64_t R, int64_t K, int B);
nm_status nm_spmv(const uint32_t *masks, const nm_bf16 *values, int64_t R, int64_t K, const nm_bf16 *x,
                  int64_t ldx, int B, nm_bf16 *y, int64_t ldy, void *workspace, size_t workspace_bytes,
                  void *hip_stream);

/*
 * nm_spmv_noalloc -- nm_spmv without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same product, same kernels and bit-identical results; the fp32
 * partial sums of split rows live in a fixed scratch array of 4 MiB that the library holds
 * on every device it runs on until the process ends.  The call allocates nothing and calls
 * no allocating routine; its first call on a device looks up that device's scratch
 * address (a host-side lookup, no allocation).
 * A shape whose split rows need more than 4 MiB of partial sums (as nm_spmv_workspace_bytes
 * would report) is rejected with NM_ERR_WORKSPACE before any HIP call; every other shape
 * of nm_spmv is accepted.  All calls on one device share its scratch: calls that overlap
 * in time on one device (different streams or threads) race and must be serialised by the
 * caller.  Arguments and the remaining conditions as for nm_spmv.
 */
nm_status nm_spmv_noalloc(const uint32_t *masks, const nm_bf16 *values, int64_t R, int64_t K, const nm_bf16 *x,
                          int64_t ldx, int B, nm_bf16 *y, int64_t ldy, void *hip_stream);

/*
 * dense_gemv -- same-GPU dense baseline for the same product with an unpruned bf16
 * matrix (decode is a memory-bound matrix-vector product [SD-cn, 前置知识 Prefill 与
 * Decoding]):  y[b][i] = sum_j W[i][j] * x[b][j], fp32 accumulate, bf16 RNE store.
 * W: bf16 [R][ldw]; x: bf16 [B][ldx]; y: bf16 [B][ldy].
 * workspace: at least dense_gemv_workspace_bytes(R, K, B) bytes (NULL if 0).
 * Requires R >= 1, K >= 8, K % 8 == 0, 1 <= B <= 8, ldw >= K, ldx >= K, ldy >= R.
 */
size_t dense_gemv_workspace_bytes(int64_t R, int64_t K, int B);
nm_status dense_gemv(const nm_bf16 *W, int64_t ldw, int64_t R, int64_t K, const nm_bf16 *x, int64_t ldx,
                     int B, nm_bf16 *y, int64_t ldy, void *workspace, size_t workspace_bytes,
                     void *hip_stream);

/*
 * nm_spmv_multi -- several packed matrices that read the same input x in one launch,
 * e.g. the q, k and v projections of an attention block, or gate and up of an MLP
 * (each is one pruned linear of the decode step [SD-cn, 方法步骤详情 第四步]).  x is
 * staged once and one grid walks the rows of all matrices; results are identical to P
 * separate nm_spmv calls with the same x (the per-row arithmetic does not change).
 * mats: HOST array of P descriptors (1 <= P <= 8), read during the call only; every
 * matrix has K columns, its own R, canonical masks/values and output y [B][ldy].
 * Total rows <= 2^30.  Workspace as for nm_spmv, sized by nm_spmv_multi_workspace_bytes.
 */
typedef struct {
    const uint32_t *masks;  /* [R][K/32] */
    const nm_bf16 *values;  /* [R][K/2]  */
    int64_t R;
    nm_bf16 *y;             /* [B][ldy], ldy >= R */
    int64_t ldy;
} nm_spmv_matrix;
size_t nm_spmv_multi_workspace_bytes(const nm_spmv_matrix *mats, int P, int64_t K, int B);
nm_status nm_spmv_multi(const nm_spmv_matrix *mats, int P, int64_t K, const nm_bf16 *x, int64_t ldx, int B,
                        void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * nm_spmv_swiglu -- the gate and up projections of a gated (SwiGLU) MLP block in one
 * launch, with the activation fused into the epilogue:
 *     h[b][i] = silu(g) * u,  g = sum_j Wgate[i][j] x[b][j],  u = sum_j Wup[i][j] x[b][j],
 *     silu(g) = g / (1 + exp(-g)),
 * for 0 <= i < R.  The models the pages evaluate (Llama-3.1-8B, Llama-3.3-70B, Qwen3)
 * use this block; each projection is one pruned linear of the decode step [SD-cn,
 * 方法步骤详情 第四步].  g and u are the fp32 row totals of the same walk as nm_spmv
 * (never rounded to bf16); silu and the product are fp32, h is rounded once to bf16.
 * Both packed matrices are R x K in the canonical layout; x: bf16 [B][ldx]; h: bf16
 * [B][ldh].  Workspace: nm_spmv_swiglu_workspace_bytes(R, K, B).  Requires R <= 2^29 and
 * the nm_spmv conditions otherwise.
 */
size_t nm_spmv_swiglu_workspace_bytes(int64_t R, int64_t K, int B);
nm_status nm_spmv_swiglu(const uint32_t *gate_masks, const nm_bf16 *gate_values, const uint32_t *up_masks,
                         const nm_bf16 *up_values, int64_t R, int64_t K, const nm_bf16 *x, int64_t ldx, int B,
                         nm_bf16 *h, int64_t ldh, void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * nm_spmv_plan / nm_spmv_multi_plan -- the launch plan that nm_spmv (epilogue
 * NM_EPI_NONE, R rows) or nm_spmv_swiglu (NM_EPI_SWIGLU, R rows of gate and of up)
 * would use on the current device, or nm_spmv_multi for P matrices of rows[0..P-1]
 * rows, with a contiguous x (ldx = K).  A test and tuning aid: host only, launches
 * nothing, and the same planner as the compute calls, so a test can check which kernel
 * instance a shape reaches.  With no visible device the planner assumes 256 compute
 * units and 160 KiB of LDS per workgroup.  Returns NM_ERR_NULL for a NULL plan (or
 * rows), NM_ERR_SHAPE / NM_ERR_PATTERN for sizes or an epilogue the compute call would
 * reject; *plan is written only on NM_OK.
 */
typedef enum { NM_EPI_NONE = 0, NM_EPI_SWIGLU = 1 } nm_epilogue;
/* NM_KERNEL_WORD_HALF_ROWS: the word-per-lane walk with every row split between two
   waves of a workgroup (one matrix, one token, rows of 7+ strips of 64 words).
   NM_KERNEL_WORD_STRIPS: the word-per-lane walk with each workgroup owning consecutive
   rows and dealing their 64-word strips to its waves in turn (one matrix, one token). */
typedef enum {
    NM_KERNEL_WORD = 0,
    NM_KERNEL_TILE = 1,
    NM_KERNEL_WORD_HALF_ROWS = 2,
    NM_KERNEL_WORD_STRIPS = 3
} nm_kernel_kind;
typedef struct {
    int kernel;             /* nm_kernel_kind: word-per-lane walk (whole rows, half rows or strips per
                               wave), or the matrix-core tile walk */
    int threads;            /* workgroup size */
    int grid_x;             /* workgroups per row slice (word) / resident workgroups (tile) */
    int splits;             /* row slices; > 1: fp32 partial sums and an ordered second pass */
    int tiles_per_step;     /* tile walk: 16-row tiles sharing one x operand (1 or 2); 0 otherwise */
    int x_steps_in_registers; /* tile walk: steps whose x operand each wave holds in registers for the
                                 whole launch (its steps then load weights only); 0: x re-read per step */
    int rows_per_group;     /* strip walk: consecutive rows owned by one workgroup; 0 otherwise */
    size_t lds_bytes;       /* dynamic LDS of the word-per-lane walk per workgroup */
    size_t workspace_bytes; /* what the compute call requires */
} nm_launch_plan;
nm_status nm_spmv_plan(int64_t R, int64_t K, int B, int epilogue, nm_launch_plan *plan);
nm_status nm_spmv_multi_plan(const int64_t *rows, int P, int64_t K, int B, nm_launch_plan *plan);

/* dense_gemv_swiglu -- the dense baseline of nm_spmv_swiglu: unpruned bf16 gate and up
 * matrices W_gate, W_up [R][ldw], same epilogue and conventions. */
size_t dense_gemv_swiglu_workspace_bytes(int64_t R, int64_t K, int B);
nm_status dense_gemv_swiglu(const nm_bf16 *W_gate, const nm_bf16 *W_up, int64_t ldw, int64_t R, int64_t K,
                            const nm_bf16 *x, int64_t ldx, int B, nm_bf16 *h, int64_t ldh, void *workspace,
                            size_t workspace_bytes, void *hip_stream);

/* dense_gemv_multi -- the dense baseline for the same grouping (same conventions). */
typedef struct {
    const nm_bf16 *W;  /* [R][ldw] */
    int64_t ldw;
    int64_t R;
    nm_bf16 *y;        /* [B][ldy] */
    int64_t ldy;
} dense_matrix;
size_t dense_gemv_multi_workspace_bytes(const dense_matrix *mats, int P, int64_t K, int B);
nm_status dense_gemv_multi(const dense_matrix *mats, int P, int64_t K, const nm_bf16 *x, int64_t ldx, int B,
                           void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Index-metadata formats [SD-en, Main Findings (metadata reduction); SD-cn, 核心方法
 * (核心创新二)]: the pages price the bitmask (2 bits per kept weight at 50%) against a
 * uint8 offset (8 bits) and an int32 column index (32 bits, the nmSPARSE format) per
 * kept weight.  The library builds both index formats from a bitmask and runs the same
 * product on them so the metadata cost can be measured on one kernel design.
 *
 *   NM_META_BITMASK    uint32 [R][K/32]: the canonical masks (as nm_spmv).
 *   NM_META_U8_OFFSET  uint8  [R][K/2]:  for kept weight t of word w (the t-th set bit,
 *                      lowest first), its column minus 32w, i.e. 0..31; 16 bytes per
 *                      word, in the order of values.
 *   NM_META_I32_INDEX  int32  [R][K/2]:  the same weight's column index within the row,
 *                      32w + offset; 16 per word, in the order of values.
 */
typedef enum {
    NM_META_BITMASK = 0,
    NM_META_U8_OFFSET = 1,
    NM_META_I32_INDEX = 2
} nm_meta_format;

/*
 * nm_meta_from_mask -- converts canonical masks into NM_META_U8_OFFSET or
 * NM_META_I32_INDEX metadata (format NM_META_BITMASK is rejected with NM_ERR_PATTERN:
 * there is nothing to convert).  meta: device buffer of R*K/2 bytes (uint8) or 2*R*K
 * bytes (int32), 16-byte aligned.  Requires R >= 1, K >= 32, K % 32 == 0 and 16 set
 * bits per mask word.
 */
nm_status nm_meta_from_mask(const uint32_t *masks, int64_t R, int64_t K, int format, void *meta,
                            void *hip_stream);

/*
 * nm_spmv_meta -- nm_spmv with the metadata in any nm_meta_format: the same product
 * y[b][i] = sum_j Wsparse[i][j] * x[b][j] with the t-th kept weight of word w at the
 * column the metadata gives.  Same precision (fp32 products and sums, bf16 RNE store),
 * workspace (nm_spmv_workspace_bytes) and requirements as nm_spmv; meta must be 4-byte
 * (bitmask) or 16-byte (index formats) aligned.  Bitmask and uint8 offsets also sum in
 * nm_spmv's order (identical bits); int32 indices are walked a quarter-word per lane, a
 * different fp32 summation order (deterministic run to run).  At 50% N:M every weight of word w lies
 * in columns [32w, 32w+32); the kernel reads the low five bits of each offset/index
 * (an entry that breaks this rule reads a wrong column of the same word, never memory
 * outside x).  Unknown formats fail with NM_ERR_PATTERN.
 */
nm_status nm_spmv_meta(const void *meta, int format, const nm_bf16 *values, int64_t R, int64_t K,
                       const nm_bf16 *x, int64_t ldx, int B, nm_bf16 *y, int64_t ldy, void *workspace,
                       size_t workspace_bytes, void *hip_stream);

/*
 * 50% unstructured rows [SD-en, Methodology Steps 3-4: the pages' other 50% setting,
 * "50% unstructured sparsity", and the case the fixed-step walk does not cover].
 *
 * nm_prune_pack_unstructured -- the same Wanda score and tie rule as nm_prune_pack, with
 * the whole row as the comparison group: row i keeps the K/2 columns that come first
 * under (score descending, column ascending).  Same encoding: masks uint32 [R][K/32]
 * (bit b of word w <-> column 32w+b), values bf16 [R][K/2] in increasing column order;
 * a word may now hold 0..32 set bits, every row exactly K/2.  Alignment: W and col_norm
 * 16 bytes (ldw % 8 == 0), masks 4, values 2.
 *
 * nm_spmv_unstructured -- y[b][i] = sum_j Wsparse[i][j] * x[b][j] for such rows: each
 * word's set bits are walked lowest first and paired with the row's values in order (the
 * value offset of a word is the popcount of the row's earlier words).  Same arithmetic,
 * output rounding, shape/alignment rules and workspace protocol as nm_spmv (workspace:
 * nm_spmv_unstructured_workspace_bytes).  Requires K/2 set bits per row (not re-checked
 * on the device; a violating row gives undefined values but no access outside the
 * row's values).
 *
 * nm_unpack_unstructured -- inverse of nm_prune_pack_unstructured (zeros where bits are
 * clear); W_out bf16 [R][ldw], 16-byte aligned, ldw % 8 == 0.
 */
nm_status nm_prune_pack_unstructured(const nm_bf16 *W, int64_t ldw, int64_t R, int64_t K, const float *col_norm,
                                     uint32_t *masks, nm_bf16 *values, void *hip_stream);
size_t nm_spmv_unstructured_workspace_bytes(int64_t R, int64_t K, int B);
nm_status nm_spmv_unstructured(const uint32_t *masks, const nm_bf16 *values, int64_t R, int64_t K, const nm_bf16 *x,
                               int64_t ldx, int B, nm_bf16 *y, int64_t ldy, void *workspace, size_t workspace_bytes,
                               void *hip_stream);
nm_status nm_unpack_unstructured(const uint32_t *masks, const nm_bf16 *values, int64_t R, int64_t K, nm_bf16 *W_out,
                                 int64_t ldw, void *hip_stream);

/*
 * OBS / SparseGPT N:M solver [SD-cn, 前置知识 (训练后剪枝与OBS框架) and 方法步骤详情 第二步:
 * H = 2 X X^T, saliency w_q^2 / (2 [H^-1]_qq), compensation
 * delta_w = -(w_q / [H^-1]_qq) H^-1_{:,q}; SD-en, Methodology Step 1].  All in fp64.
 *
 * nm_hessian -- H = 2 X^T X for calibration activations X: bf16 [T][ldx] (tokens by the
 * K input channels, the layout nm_col_norm takes); H: fp64 [K][ldh], full symmetric
 * matrix.  Requires 1 <= T <= 2^30, 1 <= K <= 65536, ldx >= K, ldh >= K.
 *
 * nm_obs_inverse_factor -- U: fp64 [K][ldu], upper triangular with positive diagonal and
 * U^T U = (H + lambda I)^-1, lambda = damp * mean(diag H) (entries below the diagonal
 * are written as 0).  U[i][i]^2 is the inverse-Hessian entry of column i among the
 * columns i.. (the quantity the column-sequential solver needs).  Requires K a multiple
 * of 32 in [32, 65536], damp >= 0, H + lambda I positive definite (otherwise the
 * results are NaN; nothing faults).  Workspace: nm_obs_inverse_factor_workspace_bytes(K)
 * (about 16 K^2 bytes), 8-byte aligned.
 *
 * nm_sparsegpt_prune_pack -- the column-sequential solver (SparseGPT's schedule): columns
 * are fixed left to right; at the first column of each group of M, every row keeps the
 * N columns of largest w^2 / U[c][c]^2 (current, already compensated weights; ties keep
 * the lower column); a pruned weight moves the later columns of its row by
 * -(w / U[c][c]) * U[c][c+1:].  Output in the nm_prune_pack format (masks uint32
 * [R][K/32], values bf16 [R][K/2] in increasing column order), the kept weights being
 * the compensated ones rounded once to bf16 (nearest even).  W: bf16 [R][ldw] (not
 * modified); H as for nm_obs_inverse_factor.  Only 50% patterns (N = M/2, M in
 * {4, 8, 16, 32}).  Workspace: nm_sparsegpt_workspace_bytes(R, K) (about 16 K^2 + 8 R K
 * bytes), 8-byte aligned; values 16-byte aligned.
 */
nm_status nm_hessian(const nm_bf16 *X, int64_t T, int64_t K, int64_t ldx, double *H, int64_t ldh, void *hip_stream);
size_t nm_obs_inverse_factor_workspace_bytes(int64_t K);
nm_status nm_obs_inverse_factor(const double *H, int64_t ldh, int64_t K, double damp, double *U, int64_t ldu,
                                void *workspace, size_t workspace_bytes, void *hip_stream);
size_t nm_sparsegpt_workspace_bytes(int64_t R, int64_t K);
nm_status nm_sparsegpt_prune_pack(const nm_bf16 *W, int64_t ldw, int64_t R, int64_t K, const double *H, int64_t ldh,
                                  int N, int M, double damp, uint32_t *masks, nm_bf16 *values, void *workspace,
                                  size_t workspace_bytes, void *hip_stream);

/*
 * nm_unpack -- inverse of the packing: W_out[i][j] = kept value of column j, or +0.0
 * where the bit is clear.  W_out: bf16 [R][ldw] (ldw >= K, multiple of 8).
 * Requires R >= 1, K >= 32, K % 32 == 0 and 16 set bits per mask word.
 */
nm_status nm_unpack(const uint32_t *masks, const nm_bf16 *values, int64_t R, int64_t K, nm_bf16 *W_out,
                    int64_t ldw, void *hip_stream);

/*
 * nm_stream_read -- measurement aid, not part of the method: reads `bytes` bytes at `buf`
 * once, with the same 16-byte non-temporal loads and 512-thread workgroups as the
 * matrix-vector kernels (one workgroup per CU, 3-4 KiB in flight per wave: the fastest
 * plain read found), and writes one XOR-fold of the dwords per wave to
 * sink[0 .. nm_stream_read_sink_words(bytes)).  Timed under the same rotation of
 * distinct buffers as the SpMV, it gives the rate a kernel that only streams reaches --
 * the achievable figure the SpMV's % of the 8 TB/s peak is read against.  The XOR of all
 * sink words equals the XOR of all dwords of the buffer.
 *
 * buf: device, 16-byte aligned, caller-owned, read only.  bytes: multiple of 16 in
 * [16, 2^31] (else NM_ERR_SHAPE).  sink: device uint32 array, caller-owned, at least
 * nm_stream_read_sink_words(bytes) words (else NM_ERR_WORKSPACE).  Asynchronous on
 * hip_stream like every other entry point.
 */
size_t nm_stream_read_sink_words(size_t bytes);
nm_status nm_stream_read(const void *buf, size_t bytes, uint32_t *sink, size_t sink_words, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* NM_SPMV_H */
