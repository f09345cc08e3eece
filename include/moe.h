/*
 * moe.h -- C ABI of libmoe: one mixture-of-experts layer, forward and
 * backward, on one AMD Instinct MI355X (gfx950).
 *
 * The layer follows the pages' description of Ai2's Olmo-core 3 MoE path:
 *  - a router picks a few experts per token (deniz.in, "Hedeflediği kapasite
 *    sorunu");
 *  - routing metadata (group sizes, split sizes) stays on the GPU so the host
 *    enqueues work without waiting for a copy back (deniz.in, "Yeni stack
 *    nasıl çalışıyor"; unite.ai/hi, "पैरालेलिज़्म, प्रिसीजन, और मेमोरी तकनीकें");
 *  - each selected token row is written straight into its expert's input
 *    buffer (same sections; donmalab.com, "擴展與最佳化手段");
 *  - device-scheduled grouped GEMMs run the uneven per-expert shapes, with a
 *    padded-to-common-capacity alternative kept for comparison (deniz.in,
 *    "Yeni stack nasıl çalışıyor");
 *  - MXFP8 for the feed-forward GEMMs (bigchange.ai pt-BR, "Três números,
 *    três denominadores").
 *
 * Conventions shared by every call:
 *  - Pointers are device pointers unless a parameter says otherwise. The
 *    caller allocates and owns every buffer, workspaces included; the library
 *    never allocates, frees, synchronises or copies to the host.
 *  - Every call only enqueues kernels on `stream` and returns at once.
 *    Argument errors are detected on the host before anything is enqueued and
 *    returned as a negative moe_status; a failed launch returns MOE_ERR_HIP.
 *    Data-dependent errors (an expert id outside [0, E)) are reported through
 *    a device-resident flag that the caller reads whenever it next syncs.
 *  - Row-major storage. Element types: MOE_F32 (binary32) or MOE_BF16
 *    (bfloat16, passed as raw 16-bit patterns). Logits, gate weights, their
 *    gradients and dlogits are always binary32. Indices are int32.
 *  - Tensors of 16-bit or 32-bit elements must start 16-byte aligned, and
 *    row lengths (d, F) must be multiples of 8.
 *  - Notation: T tokens, d model dim, E experts, k experts per token, F expert
 *    hidden dim, R = T*k routed slots; slot s = t*k + j is token t's j-th
 *    choice; n_rows is the row count of the permuted buffers (R dropless,
 *    E*capacity padded).
 *  - Results are bitwise reproducible run to run: no floating-point atomics.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad size or mode */
  MOE_ERR_UNSUPPORTED = -2,  /* valid but outside the supported limits */
  MOE_ERR_WORKSPACE = -3,    /* workspace missing or too small */
  MOE_ERR_HIP = -4           /* a HIP launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Limits: 1 <= k <= min(E, 16), 1 <= E <= 1024, T*k < 2^31. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16

/* Text for a status code (static storage; never NULL). */
const char* moe_status_string(int status);

/* ABI version of this header: 6. */
int moe_abi_version(void);

/* ----------------------------------------------------------------- router
 * moe_router_gemm: logits[t,e] = sum_i x[t,i] * w_r[i,e], binary32 out.
 * The learned router of the pages' small configurations (bigchange.ai pt-BR,
 * "O que um engenheiro pode realmente testar").
 *   x [T,d] and w_r [d,E] of `dtype`; logits [T,E] binary32.
 *   Accumulation is binary32 in a fixed order (the bf16 products are exact in
 *   binary32). bf16 with E in {8, 16}, d % 256 == 0, d * E <= 32768 and w_r
 *   16-byte aligned runs on the matrix cores; the other shapes on FMA
 *   kernels with another (fixed) summation order. */
int moe_router_gemm(int dtype, const void* x, const void* w_r, int T, int d, int E,
                    float* logits, hipStream_t stream);

/* moe_route: top-k experts of each token and their gate weights.
 * The pages say only that each token goes to a few experts; the reading is a
 * softmax over all E logits, the k largest kept and renormalised to sum to 1,
 * i.e. w_j = exp(l_j - l_max) / sum over the selected exp(l_i - l_max).
 * Selection compares the binary32 logits (softmax is increasing); equal
 * logits, +0 and -0 included, go to the lower expert id; slot j holds the
 * j-th largest. NaN logits give unspecified (but in-range) results.
 *   logits [T,E] binary32 -> topk_idx [T,k] int32, topk_w [T,k] binary32. */
int moe_route(const float* logits, int T, int E, int k, int32_t* topk_idx, float* topk_w,
              hipStream_t stream);

/* ----------------------------------------------------------------- metadata
 * moe_offsets: GPU-resident routing metadata (deniz.in, "Yeni stack nasıl
 * çalışıyor": split and group sizes never leave the GPU).
 * Rows are expert-major and, within an expert, in slot order (a stable
 * counting sort of the flat expert ids):
 *   counts[E]      slots routed to each expert (before any drop)
 *   offsets[E+1]   exclusive prefix sum of counts; offsets[E] = R
 *   row_of[R]      dropless (capacity == 0): offsets[e] + rank of the slot
 *                  among e's slots; padded (capacity C > 0): e*C + rank if
 *                  rank < C, else -1 (dropped: overflow goes in slot order)
 *   src_slot[n]    inverse of row_of over n_rows = R (dropless) or E*C
 *                  (padded) rows; -1 on pad rows
 *   n_dropped[1]   number of dropped slots (0 when dropless)
 *   err_flag[1]    set to 1 if any expert id is outside [0, E) (those slots
 *                  get row_of = -1 and are not counted); left untouched
 *                  otherwise, so the caller zeroes it once and may check it
 *                  after any number of calls.
 * ws: workspace of at least moe_offsets_workspace_bytes(T, k, E) bytes. */
size_t moe_offsets_workspace_bytes(int T, int k, int E);
int moe_offsets(const int32_t* topk_idx, int T, int k, int E, int capacity, int32_t* counts,
                int32_t* offsets, int32_t* row_of, int32_t* src_slot, int32_t* n_dropped,
                int32_t* err_flag, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_offsets_noalloc: moe_offsets without a caller workspace and without
 * any device allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Same arguments (minus ws, ws_bytes), results and errors as
 * moe_offsets; the workspace is a static array of the library, one per GPU,
 * MOE_OFFSETS_NOALLOC_MAX_BYTES long, held until the process ends. Calls whose
 * moe_offsets_workspace_bytes(T, k, E) exceeds it return MOE_ERR_UNSUPPORTED
 * (1 MiB: e.g. T*k up to 2M slots at E = 128, 256K slots at E = 1024).
 * All calls on one GPU share that GPU's array: calls that overlap on one GPU
 * (on different streams, or from different threads without ordering) race;
 * calls ordered on one stream do not. A failure to resolve the array's
 * device address returns MOE_ERR_HIP. */
#define MOE_OFFSETS_NOALLOC_MAX_BYTES ((size_t)1 << 20)
int moe_offsets_noalloc(const int32_t* topk_idx, int T, int k, int E, int capacity, int32_t* counts,
                        int32_t* offsets, int32_t* row_of, int32_t* src_slot, int32_t* n_dropped,
                        int32_t* err_flag, hipStream_t stream);

/* ----------------------------------------------------------------- row movement
 * moe_permute: x_perm[row_of[s]] = x[s / k] for every kept slot s: each
 * selected token row is written straight into its expert's rows (unite.ai/hi,
 * "पैरालेलिज़्म, प्रिसीजन, और मेमोरी तकनीकें"). If src_slot is not NULL, every row r
 * with src_slot[r] == -1 (a pad row of the padded layout) is zero-filled;
 * src_slot may be NULL only when n_rows == T*k (dropless: all rows are hit).
 *   x [T,d], x_perm [n_rows,d] of `dtype`. Row ids outside [0, n_rows) are
 *   skipped. */
int moe_permute(int dtype, const void* x, int T, int d, int k, const int32_t* row_of,
                const int32_t* src_slot, int n_rows, void* x_perm, hipStream_t stream);

/* moe_unpermute_combine: y[t] = y_add[t] + sum_j w[t,j] * y_perm[row_of[t,j]],
 * binary32 accumulation in slot order j = 0..k-1, one rounding to `dtype`;
 * dropped slots (row -1) add nothing. Reading: the gate weight scales each
 * expert's output after the down projection. y_add (may be NULL) is the
 * shared expert's output, which the pages' production configurations add to
 * the routed experts' (bigchange.ai pt-BR, "O que um engenheiro pode
 * realmente testar").
 *   y_perm [n_rows,d], y_add and y [T,d] of `dtype`; topk_w [T,k] binary32. */
int moe_unpermute_combine(int dtype, const void* y_perm, const int32_t* row_of,
                          const float* topk_w, int T, int k, int d, int n_rows,
                          const void* y_add, void* y, hipStream_t stream);

/* moe_unpermute_combine_bwd: derived, the adjoint of moe_unpermute_combine
 * (its chain rule with respect to y_perm and the gate weights).
 *   dy_perm[row_of[t,j]] = w[t,j] * dy[t]   (rounded once to `dtype`)
 *   dtopk_w[t,j] = <dy[t], y_perm[row_of[t,j]]>  (binary32; 0 if dropped)
 * If src_slot is not NULL, pad rows (src_slot == -1) of dy_perm are zeroed
 * and the work runs in row order (row r from slot src_slot[r]: dy_perm
 * written and y_perm read in address order, faster than token order, same
 * results bit for bit); src_slot must then be the one moe_offsets wrote with
 * row_of. src_slot may be NULL only when n_rows == T*k. */
int moe_unpermute_combine_bwd(int dtype, const void* dy, const void* y_perm,
                              const float* topk_w, const int32_t* row_of,
                              const int32_t* src_slot, int T, int k, int d, int n_rows,
                              void* dy_perm, float* dtopk_w, hipStream_t stream);

/* moe_permute_bwd: derived, the adjoint of moe_permute (each token row
 * receives the sum of its routed rows' gradients),
 *   dx[t] = dx_add[t] + sum_j dx_perm[row_of[t,j]]  (+ sum_e dlogits[t,e] * w_r[:,e])
 * binary32 accumulation, one rounding to `dtype`. The router term is added
 * when dlogits and w_r are not NULL (learned router); it is the router
 * GEMM's share of dx, folded in so that dx is written once. dx_add (may be
 * NULL) is the shared expert's share of dx.
 *   dx_perm [n_rows,d], dx_add and dx [T,d], w_r [d,E] of `dtype`;
 *   dlogits [T,E] f32. */
int moe_permute_bwd(int dtype, const void* dx_perm, const int32_t* row_of, int T, int k, int d,
                    int n_rows, const float* dlogits, const void* w_r, int E, const void* dx_add,
                    void* dx, hipStream_t stream);

/* ----------------------------------------------------------------- router backward
 * moe_route_bwd: derived, the adjoint of moe_route with the selection held
 * fixed (the chain rule of the renormalised top-k softmax), dlogits through
 * the gate: for selected e_j, dl = w_j (dw_j - sum_i w_i dw_i);
 * exactly 0 for unselected experts.
 *   topk_idx, topk_w, dtopk_w [T,k] -> dlogits [T,E] binary32. */
int moe_route_bwd(const int32_t* topk_idx, const float* topk_w, const float* dtopk_w, int T,
                  int E, int k, float* dlogits, hipStream_t stream);

/* moe_router_gemm_bwd: derived, the adjoint of moe_router_gemm with respect
 * to w_r (its share of dx is added by moe_permute_bwd):
 * dw_r = x^T dlogits, binary32 accumulation over tokens
 * in a fixed order, one rounding to `dtype`. bf16 with E <= 16, E % 4 == 0,
 * d % 256 == 0 and x and dlogits 16-byte aligned runs on the matrix cores
 * with each dlogits value carried as two bf16 terms (hi = bf16(v), lo =
 * bf16(v - hi)): the products are within 2^-16 of x * dlogits relative to
 * it, far below the final bf16 rounding.
 *   x [T,d], dw_r [d,E] of `dtype`; dlogits [T,E] binary32;
 *   ws of at least moe_router_bwd_workspace_bytes(T, d, E) bytes. */
size_t moe_router_bwd_workspace_bytes(int T, int d, int E);
int moe_router_gemm_bwd(int dtype, const void* x, const float* dlogits, int T, int d, int E,
                        void* dw_r, void* ws, size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------------------- grouped GEMM
 * moe_grouped_gemm: the expert GEMMs over the uneven per-expert row blocks
 * ("device-scheduled grouped GEMM", deniz.in, "Yeni stack nasıl çalışıyor").
 * Expert e owns rows [group_offsets[e], group_offsets[e+1]) of the permuted
 * buffers (dropless), or rows [e*capacity, (e+1)*capacity) when capacity > 0
 * (the padded comparison path). Group sizes are read on the device only.
 * All products accumulate in binary32 and each output is rounded once to
 * `dtype`. Expert FFN reading (the pages name no activation): SwiGLU without
 * biases, H = silu(X Wg) * (X Wu), Y = H Wd.
 *
 *   op                     reads                        writes
 *   MOE_GG_FWD_GATE_UP     x_perm, w_gate, w_up         g, u, h    (h from the
 *                                                       rounded g and u; g and
 *                                                       u may both be NULL:
 *                                                       then only h is written,
 *                                                       the forward of a layer
 *                                                       that recomputes g and u
 *                                                       in its backward)
 *   MOE_GG_FWD_DOWN        h, w_down                    y_perm
 *   MOE_GG_DGRAD_DOWN      dy_perm, w_down, g, u        dg, du:  dH = dY Wd^T,
 *                          s = sigmoid(g), dg = dH*u*s*(1+g*(1-s)), du = dH*g*s
 *   MOE_GG_DGRAD_GATE_UP   dg, du, w_gate, w_up         dx_perm = dg Wg^T + du Wu^T
 *   MOE_GG_WGRAD_DOWN      h, dy_perm                   dw_down[e] = H_e^T dY_e
 *   MOE_GG_WGRAD_GATE_UP   x_perm, dg, du               dw_gate[e] = X_e^T dG_e,
 *                                                       dw_up[e] = X_e^T dU_e
 * Shapes: x_perm, y_perm, dy_perm, dx_perm [n_rows,d]; g, u, h, dg, du
 * [n_rows,F]; w_gate, w_up, dw_gate, dw_up [E,d,F]; w_down, dw_down [E,F,d].
 * Weight gradients of experts with no rows are written as zeros. Rows outside
 * every group are neither read nor written. The bf16 matrix-core path (d and
 * F multiples of 256) addresses each operand with 32-bit byte offsets:
 * n_rows * max(d, F) * 2 and d * F * 2 must stay below 2^31, otherwise the
 * call returns MOE_ERR_UNSUPPORTED (binary32 and other shapes run a plain
 * FMA kernel without this limit). The host cannot see the group
 * sizes: offsets must be non-decreasing with group_offsets[E] <= n_rows
 * (each group is clamped to [0, n_rows] on the device).
 * ws: moe_grouped_gemm_workspace_bytes(desc) bytes, 4-byte aligned,
 * device memory owned by the caller. The weight gradients over
 * device-resident groups (capacity == 0) need at least 64 bytes, 4-byte
 * aligned (else MOE_ERR_WORKSPACE): the call writes there how the launch
 * splits its tiles over the chip, computed on the device from the group sizes
 * (tiles of the experts with the most rows carry the most work). A bf16
 * matrix-core weight gradient with fewer than 512 output tiles (128 x 256
 * outputs each; 128 x 128 per matrix for the gate/up pair, e.g. a shared
 * expert, E == 1) would leave compute units idle: when the workspace holds
 * the size this function reports and is 16-byte aligned, the call splits each
 * expert's rows (K) into min(8, ceil(512 / tiles)) chunks of whole 32-row
 * steps, writes each chunk's binary32 sums from byte 256 of the workspace
 * ([chunk][E][M][N] floats, M x N the gradient's shape; the gate/up pair as
 * one [d][2F] block) and adds the chunks in chunk order before one rounding
 * to bf16, so the result is deterministic; with a workspace of 64 bytes up to
 * that size the same call runs K unsplit. The other ops need no workspace.
 * Calls sharing one workspace must be ordered on one stream. */
typedef enum {
  MOE_GG_FWD_GATE_UP = 0,
  MOE_GG_FWD_DOWN = 1,
  MOE_GG_DGRAD_DOWN = 2,
  MOE_GG_DGRAD_GATE_UP = 3,
  MOE_GG_WGRAD_DOWN = 4,
  MOE_GG_WGRAD_GATE_UP = 5
} moe_gg_op;

typedef struct moe_gg_desc {
  int op;                        /* moe_gg_op */
  int dtype;                     /* MOE_F32 or MOE_BF16 */
  int E, d, F;                   /* experts, model dim, expert hidden dim */
  int n_rows;                    /* rows of the permuted activations */
  int capacity;                  /* 0: groups from group_offsets; > 0: uniform */
  const int32_t* group_offsets;  /* [E+1], device; unused when capacity > 0 */
  void* x_perm;
  void* g;
  void* u;
  void* h;
  void* y_perm;
  void* dy_perm;
  void* dg;
  void* du;
  void* dx_perm;
  void* w_gate;
  void* w_up;
  void* w_down;
  void* dw_gate;
  void* dw_up;
  void* dw_down;
  void* ws;
  size_t ws_bytes;
} moe_gg_desc;

size_t moe_grouped_gemm_workspace_bytes(const moe_gg_desc* desc);
int moe_grouped_gemm(const moe_gg_desc* desc, hipStream_t stream);

/* ----------------------------------------------------------------- MXFP8
 * The pages credit MXFP8 for most of the feed-forward speed-up (bigchange.ai
 * pt-BR, "Três números, três denominadores"; unite.ai/hi, "पैरालेलिज़्म,
 * प्रिसीजन, और मेमोरी तकनीकें") but fix no format. Reading, per the public OCP
 * Microscaling Formats v1.0 specification: blocks of 32 consecutive values
 * along each GEMM's contraction axis share one E8M0 scale byte (value
 * 2^(code-127)); elements are E4M3 bytes (bias 7, largest 448, subnormals
 * m*2^-9, no infinities). For a block with largest magnitude amax the scale
 * exponent is X = clamp(floor(log2 amax) - 8, -127, 127) (X = -127 for an
 * all-zero block) and each element is v * 2^-X rounded to nearest-even and
 * saturated to +-448, keeping the sign bit (also when it rounds to zero).
 * Code 0xFF (NaN) is never written.
 *
 * moe_mx_quantize: bf16 src [rows, cols] -> E4M3 codes + E8M0 scales.
 * The quantised operand is a matrix of R rows whose K values (the GEMM's
 * contraction) run along each row: codes q [R, K], one byte per value, and
 * scales in groups of four: the scale of block b (values 32b..32b+31) of
 * row r is byte 4 * (R * (b / 4) + r) + b % 4 of s (R * K / 32 bytes). So
 * the four scales of 128 consecutive values of a row share one 4-byte word,
 * and the words of one 128-value column group are contiguous over the rows,
 * which lets a GEMM fetch the scales of many rows with one contiguous load.
 *   axis 0: blocks along each row: R = rows, K = cols; cols % 128 == 0;
 *           group_offsets must be NULL and col_stride 0.
 *   axis 1: blocks along the rows of each group, written transposed:
 *           R = cols, K = col_stride. Group g (rows [group_offsets[g],
 *           group_offsets[g+1]) of src; when group_offsets is NULL, n_groups
 *           equal groups of rows/n_groups rows) becomes K columns
 *           [p_g, p_g + ceil(n_g/128)*128) with p_g = 128 * sum_{h<g}
 *           ceil(n_h/128). Blocks restart at each group's first row; the
 *           columns past a group's last row are written as zero codes with
 *           scale code 0. Columns past the last group's segment are not
 *           written. col_stride must be a multiple of 128 and at least
 *           moe_mx_col_stride(rows, n_groups) when the offsets are on the
 *           device (a bound that holds whatever the group sizes), or
 *           n_groups * ceil(rows/n_groups/128)*128 for equal groups
 *           (rows % n_groups == 0); cols % 64 == 0.
 *   src and q 16-byte aligned, s 4-byte aligned. rows may be 0. */
int moe_mx_col_stride(int rows, int n_groups);

/* moe_mx_quantize_both: both orientations of moe_mx_quantize from one read of
 * src: q_rows/s_rows as axis 0 and q_cols/s_cols as axis 1 with the same
 * groups and col_stride (each GEMM operand of the expert layer is needed in
 * both: by rows for one GEMM, by token columns for a weight gradient).
 * cols % 128 == 0. Rows outside every group are written in neither. */
int moe_mx_quantize_both(const void* src, int rows, int cols, const int32_t* group_offsets, int n_groups,
                         int col_stride, void* q_rows, void* s_rows, void* q_cols, void* s_cols,
                         hipStream_t stream);
int moe_mx_quantize(const void* src, int rows, int cols, int axis, const int32_t* group_offsets,
                    int n_groups, int col_stride, void* q, void* s, hipStream_t stream);

/* moe_permute_mx: the permute of a dropless routed layer fused with the
 * MXFP8 quantisation of its output ("quantise on dispatch": the pages credit
 * MXFP8 with speeding up the movement of rows between experts as well as the
 * GEMMs, unite.ai/hi, "पैरालेलिज़्म, प्रिसीजन, और मेमोरी तकनीकें"). Permuted
 * row r holds x[src_slot[r] / k]; the rows are never written in bf16, only
 * quantised, in both orientations of moe_mx_quantize_both with the experts
 * as groups: q_rows/s_rows [n_rows, d] (blocks along d) and q_cols/s_cols
 * [d, col_stride] (blocks along each expert's rows).
 *   x [T,d] bf16; src_slot [n_rows] and group_offsets [E+1] on the device, as
 *   written by moe_offsets; n_rows == T*k; d % 128 == 0; col_stride as for
 *   moe_mx_quantize_both with device offsets. */
int moe_permute_mx(const void* x, int T, int d, int k, const int32_t* src_slot,
                   const int32_t* group_offsets, int E, int n_rows, int col_stride, void* q_rows,
                   void* s_rows, void* q_cols, void* s_cols, hipStream_t stream);

/* moe_grouped_gemm_mx: the six expert GEMMs of moe_grouped_gemm with every
 * operand MXFP8 (blocks of 32 along that GEMM's contraction), binary32
 * accumulation of the exact block products on the matrix cores, and bf16
 * outputs rounded once, with the same SwiGLU epilogues. Dropless groups only
 * (group_offsets [E+1] on the device). Each operand is a (codes, scales)
 * pair from moe_mx_quantize; "rows" means axis 0, "cols" axis 1 with the
 * experts as groups and token stride col_stride:
 *
 *   op                    a0            a1        b0                    b1            out0, out1, out2
 *   FWD_GATE_UP  K=d      x_perm rows   -         w_gate as [E*d,F] cols w_up likewise g, u, h
 *                                                  (groups of d rows; col_stride E*d)
 *   FWD_DOWN     K=F      h rows        -         w_down as [E*F,d] cols -             y_perm
 *                                                  (groups of F rows; col_stride E*F)
 *   DGRAD_DOWN   K=d      dy_perm rows  -         w_down as [E*F,d] rows -             dg, du (reads bf16 g, u)
 *   DGRAD_GATE_UP K=2F    dg rows       du rows   w_gate as [E*d,F] rows w_up likewise dx_perm
 *   WGRAD_DOWN   K=n_e    h cols        -         dy_perm cols           -             dw_down
 *   WGRAD_GATE_UP K=n_e   x_perm cols   -         dg cols                du cols       dw_gate, dw_up
 *
 * Shapes of the bf16 tensors are those of moe_grouped_gemm. d % 256 == 0 and
 * F % 256 == 0. Weight gradients of experts with no rows are zeros.
 *
 * ws: at least moe_grouped_gemm_mx_workspace_bytes(desc) bytes, 4-byte
 * aligned, device memory owned by the caller; MOE_ERR_WORKSPACE when missing,
 * too small or misaligned. The weight gradients need 4 * (E + 16) bytes: the call
 * writes there the tile split of moe_grouped_gemm's weight gradients and each
 * expert's first padded token column; the other ops need none. Calls sharing
 * one workspace must be ordered on one stream. */
typedef struct moe_mx_tensor {
  const void* q;   /* E4M3 codes */
  const void* s;   /* E8M0 scales */
} moe_mx_tensor;

typedef struct moe_mx_gg_desc {
  int op;                        /* moe_gg_op */
  int E, d, F;
  int n_rows;                    /* rows of the permuted activations */
  int col_stride;                /* token stride of the "cols" operands (weight gradients) */
  const int32_t* group_offsets;  /* [E+1], device */
  moe_mx_tensor a0, a1, b0, b1;
  const void* g;                 /* bf16 [n_rows,F], read by DGRAD_DOWN */
  const void* u;
  void* out0;
  void* out1;
  void* out2;
  void* ws;                      /* workspace, see above */
  size_t ws_bytes;
  /* Optional MXFP8 copies written by the epilogue from the rounded bf16
   * outputs, exactly as moe_mx_quantize_both would write them from those
   * outputs (with the experts as groups and col_stride): FWD_GATE_UP: H in
   * qo0_rows [n_rows, F] and qo0_cols [F, col_stride]; DGRAD_DOWN: dG in
   * qo0_*, dU in qo1_*. All NULL (nothing written) or all of the op's set;
   * other ops take none. This fuses the quantisation of the next GEMMs'
   * operands into the GEMM that produces them. With the copies given, the
   * bf16 tensor they are made from may be left out: out2 (H) NULL for
   * FWD_GATE_UP, or out0 and out1 (dG, dU) both NULL for DGRAD_DOWN; the
   * copies are the same either way (they come from the rounded values). */
  moe_mx_tensor qo0_rows, qo0_cols, qo1_rows, qo1_cols;
} moe_mx_gg_desc;

size_t moe_grouped_gemm_mx_workspace_bytes(const moe_mx_gg_desc* desc);
int moe_grouped_gemm_mx(const moe_mx_gg_desc* desc, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
