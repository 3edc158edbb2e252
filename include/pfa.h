/*
 * pfa.h -- C ABI of the MI355X (gfx950) progressive focused attention (PFA)
 * layer library, libpfa.so.
 *
 * A PFA layer (sources: "Progressive Focused Transformer for Single Image
 * Super-Resolution" paper notes, sections "Progressive attention across layers",
 * "Sparse matrix multiplication" and "Progressive focused resource allocation
 * strategy"; "From Local Windows to Adaptive Candidates via Individualized
 * Exploratory", individualized-attention paragraph) maps
 *     (Q, K, V, I^{l-1}, A^{l-1})  ->  (I^l, A^l, O)
 * per window-head: scaled scores q_i.k_j / sqrt(d) only over the candidate
 * list I^{l-1}(i), a softmax over that list, the Hadamard product with
 * A^{l-1}, an L1 row normalisation, the K^l largest entries kept (ties to the
 * lower slot index j), a second row normalisation, and O_i = sum_j A_ij v_j.
 * The first layer is dense in-window softmax attention (K^1 = N).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are dense, C-contiguous, and live in device memory of the current HIP
 * device; the caller allocates all of them. The layer calls never allocate,
 * free or synchronise: they validate the arguments, enqueue kernels on
 * `stream` (a hipStream_t; NULL = the null stream) and return. (Only the
 * optional timing calls at the end of this header create HIP events; the
 * backward passes take their scratch memory as a caller-owned workspace, or,
 * in pfa_dense_layer_backward_noalloc, from a static device array.)
 *
 *   Q, K, V   [B, heads, H, W, d], element type `dtype` (fp32, or bf16 bits).
 *   O         [B, heads, H, W, d] fp32.
 *   window mode (win > 0): N = win*win tokens per window, nwin = (H/win)*(W/win)
 *     windows; slot t of window (a, b) is pixel
 *       ((a*win + t/win + shift) mod H, (b*win + t%win + shift) mod W),
 *     i.e. the cyclic shift is applied by index remap, never by moving data.
 *     I and A rows are indexed [B, heads, H/win, W/win, N, K] and hold slot
 *     indices j in [0, N). I/A are passed slot-for-slot from layer to layer.
 *   global mode (win = 0): one window of N = H*W tokens per (image, head),
 *     slot = raster index y*W + x; I and A rows are [B, heads, N, K].
 *
 * Output rows of I^l list the kept candidates in their I^{l-1} order (as a
 * subsequence), with A^l aligned; each A^l row sums to 1.
 *
 * Preconditions (not checked on the device): I^{l-1} values lie in [0, N) and
 * are distinct within a row; A^{l-1} entries are finite, >= 0, and each row
 * has a positive entry; outputs do not alias inputs.
 *
 * Errors: every entry point returns PFA_OK (0) or a negative code; nothing is
 * enqueued when a code other than PFA_OK / PFA_ERR_HIP is returned.
 * PFA_ERR_HIP reports a failed launch (hipGetLastError after the launch).
 */
#ifndef PFA_H
#define PFA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PFA_OK 0
#define PFA_ERR_INVALID (-1)     /* inconsistent sizes, NULL where required */
#define PFA_ERR_UNSUPPORTED (-2) /* valid, but outside what the kernels handle */
#define PFA_ERR_HIP (-3)         /* the HIP runtime reported an error */
#define PFA_ERR_TOO_LARGE (-4)   /* exceeds the static scratch memory of a no-allocation entry point */

/* Size of the static scratch array behind the no-allocation entry point
 * (pfa_dense_layer_backward_noalloc): 16 MiB per GPU, one fp32 per query slot, so
 * at most 4194304 query slots (B * heads * (H/win) * (W/win) * win^2) per call. */
#define PFA_STATIC_SCRATCH_BYTES (16 * 1024 * 1024)

typedef enum { PFA_F32 = 0, PFA_BF16 = 1 } pfa_dtype;

typedef struct {
    int32_t B, heads, H, W, d; /* d must be 16 or 32 */
    int32_t win;               /* window side (N = win*win <= 1024), 0 = global mode */
    int32_t shift;             /* cyclic shift in [0, win); 0 in global mode */
    int32_t dtype;             /* pfa_dtype of Q, K and V */
} pfa_shape;

/*
 * Dense first layer (window mode only): softmax(q_i.k_j / sqrt(d)) over all N
 * slots of the window ("Progressive focused resource allocation strategy":
 * the first layer keeps every token and computes the complete map).
 *
 * K1 == N:  A_out  [B, heads, nwin, N, N] fp32 or NULL (then the map is not
 *                  written: O-only mode);
 *           I_out  [B, heads, nwin, N, N] int32 or NULL (row i is 0..N-1);
 *           O_out  required. Needs win to be a multiple of 4.
 *           lse_out [B, heads, nwin, N] fp32 or NULL: ln sum_j exp(q_i.k_j/sqrt(d)),
 *                  the log of row i's softmax denominator (what O-only callers
 *                  keep instead of the map: A_ij = exp(s_ij - lse_i)).
 * K1 <  N:  the K1 largest weights are kept and renormalised (as in a sparse
 *           layer whose previous map is all ones); I_out and A_out
 *           [.., N, K1] are required; lse_out must be NULL.
 * Errors: PFA_ERR_INVALID for K1 outside [1, N], NULL Q/K/V/O, NULL I_out or
 * A_out when K1 < N, H or W not a multiple of win, shift outside [0, win);
 * PFA_ERR_UNSUPPORTED for win == 0, win > 32, win not a multiple of 4 when
 * K1 == N, d not 16/32, unknown dtype, lse_out with K1 < N.
 */
int pfa_dense_layer(const pfa_shape* shape, const void* Q, const void* K, const void* V,
                    int32_t K1, int32_t* I_out, float* A_out, float* lse_out, float* O_out, void* stream);

/*
 * Sparse layer l > 1 ("Sparse matrix multiplication": scores only where
 * I^{l-1}(i, j) = 1; keep the top K^l).
 *
 * I_prev  [B, heads, nwin, N, K_prev] int32, or [B, 1, nwin, N, K_prev] when
 *         i_prev_shared != 0 (one index matrix for every head), or NULL:
 *         every slot 0..N-1 in order (then K_prev must equal N).
 * A_prev  [B, heads, nwin, N, K_prev] fp32, or NULL (all ones: plain softmax
 *         over the candidate list, e.g. the global individualized attention).
 * K_l     kept per row, 1 <= K_l <= K_prev <= min(N, 1024).
 * I_out, A_out  [B, heads, nwin, N, K_l] int32 / fp32, required.
 * O_out   [B, heads, H, W, d] fp32, required.
 * Errors: PFA_ERR_INVALID for inconsistent sizes or NULL outputs;
 * PFA_ERR_UNSUPPORTED for d not 16/32, win > 32, K_prev > 1024, N >= 2^24 in
 * global mode, unknown dtype.
 */
int pfa_sparse_layer(const pfa_shape* shape, const void* Q, const void* K, const void* V,
                     const int32_t* I_prev, int32_t i_prev_shared, const float* A_prev,
                     int32_t K_prev, int32_t K_l, int32_t* I_out, float* A_out, float* O_out,
                     void* stream);

/*
 * The same two layer calls with a relative position bias in the score
 * ("Progressive Focused Transformer" notes describe the network as relative
 * position bias based; IET applies relative positional encoding in its first
 * block): s_ij = q_i.k_j / sqrt(d) + bias[h][(dy + win - 1)(2 win - 1) + dx + win - 1]
 * with (dy, dx) = (i/win - j/win, i%win - j%win), the window-local offset of
 * slot i from slot j (the same under every cyclic shift).
 *
 * bias    [heads, (2 win - 1)^2] fp32 device table of this layer, or NULL (then
 *         the calls are exactly pfa_dense_layer / pfa_sparse_layer). Window mode
 *         only. With a bias, the sparse layer whose candidate list is every
 *         slot scores by gathers instead of MFMA.
 * Errors: as pfa_dense_layer / pfa_sparse_layer, and PFA_ERR_UNSUPPORTED for a
 * bias in global mode or, in pfa_dense_layer_rpb with K1 == N, win not a
 * multiple of 16.
 */
int pfa_dense_layer_rpb(const pfa_shape* shape, const void* Q, const void* K, const void* V, const float* bias,
                        int32_t K1, int32_t* I_out, float* A_out, float* lse_out, float* O_out, void* stream);
int pfa_sparse_layer_rpb(const pfa_shape* shape, const void* Q, const void* K, const void* V, const float* bias,
                         const int32_t* I_prev, int32_t i_prev_shared, const float* A_prev,
                         int32_t K_prev, int32_t K_l, int32_t* I_out, float* A_out, float* O_out,
                         void* stream);

/*
 * The first two layers of a chain fused, with the first layer's map never
 * written to memory. Computes what pfa_dense_layer (K1 = N) followed by
 * pfa_sparse_layer (I_prev = NULL, A_prev = that map, K_l = K2_keep) compute,
 * using the closed form of the chain ("Progressive attention across layers":
 * A^2 = Norm(A^1 (.) A_cal^2) with both maps softmaxes, so the second layer
 * keeps the top K2_keep of exp(s1_ij + s2_ij) and A^2 is that quantity
 * renormalised over the kept set).
 *
 * shape   B, heads, H, W, d, win, dtype of both layers; shape->shift must be 0,
 *         the two layers' shifts are shift1 and shift2 (each in [0, win)).
 * Q1, K1, V1 / Q2, K2, V2   the two layers' inputs, [B, heads, H, W, d].
 * O1_out  [B, heads, H, W, d] fp32: layer 1's output (required).
 * lse1_out [B, heads, nwin, N] fp32 or NULL: layer 1's log softmax denominators.
 * I2_out, A2_out  [B, heads, nwin, N, K2_keep] int32 / fp32; O2_out as O1_out.
 * Window mode with win = 32 (N = 1024) only; both layers' K must fit in LDS
 * together: bf16 (d = 16, 32) and fp32 with d = 16.
 * Errors: PFA_ERR_INVALID for NULL inputs or outputs, shifts outside [0, win),
 * shape->shift != 0, K2_keep outside [1, N]; PFA_ERR_UNSUPPORTED for global mode,
 * win != 32, fp32 with d = 32, d not 16/32, unknown dtype.
 */
int pfa_first_two_layers(const pfa_shape* shape, int32_t shift1, int32_t shift2, const void* Q1,
                         const void* K1, const void* V1, const void* Q2, const void* K2, const void* V2,
                         int32_t K2_keep, float* lse1_out, float* O1_out, int32_t* I2_out, float* A2_out,
                         float* O2_out, void* stream);

/*
 * Backward pass of the first two layers computed by pfa_first_two_layers, which
 * never writes the first layer's map A^1. Gives what pfa_sparse_layer_backward
 * (I_prev = NULL, A_prev = A^1) followed by pfa_dense_layer_backward (dA = that
 * call's dA_prev) give for the unfused pair: A^1 is recomputed at the second
 * layer's kept slots only, from Q1, K1 and lse1 (A^1_ij = exp(s1_ij - lse1_i)).
 *
 * shape, shift1, shift2, Q1..V2, K2_keep  as the forward call (window mode;
 *         shape->shift must be 0).
 * lse1    [B, heads, nwin, N] fp32: the forward's lse1_out.
 * I2, A2  [B, heads, nwin, N, K2_keep]: the forward's I2_out, A2_out.
 * dO1, dO2  [B, heads, H, W, d] fp32 gradients of O1 and O2.
 * dA2     [B, heads, nwin, N, K2_keep] fp32 gradient of A2, or NULL (zero).
 * dQ1..dV2  [B, heads, H, W, d] fp32 outputs, every element written.
 * workspace  at least pfa_first_two_layers_backward_workspace() bytes: per
 *         window-head A^1 and dA^1 at the kept slots ([N, K2_keep] fp32 each) and
 *         the dense dA^1 ([N, N] fp32), then the two single-layer passes' workspaces.
 * Deterministic, as the single-layer calls.
 * Errors: PFA_ERR_INVALID for NULL required pointers, shifts outside [0, win),
 * shape->shift != 0, K2_keep outside [1, N], a small workspace;
 * PFA_ERR_UNSUPPORTED for global mode, win % 8 != 0, K2_keep > 256, and the
 * limits of the single-layer backward calls.
 */
int pfa_first_two_layers_backward(const pfa_shape* shape, int32_t shift1, int32_t shift2, const void* Q1,
                                  const void* K1, const void* V1, const void* Q2, const void* K2, const void* V2,
                                  int32_t K2_keep, const float* lse1, const int32_t* I2, const float* A2,
                                  const float* dO1, const float* dO2, const float* dA2, float* dQ1, float* dK1,
                                  float* dV1, float* dQ2, float* dK2, float* dV2, void* workspace,
                                  int64_t workspace_bytes, void* stream);

/* Workspace bytes pfa_first_two_layers_backward needs, or a negative error code
 * (shape errors, PFA_ERR_UNSUPPORTED for global mode, PFA_ERR_INVALID for K2_keep
 * outside [1, N]). Host only. */
int64_t pfa_first_two_layers_backward_workspace(const pfa_shape* shape, int32_t K2_keep);

/*
 * Backward pass of a sparse layer ("Progressive attention across
 * layers" and "Sparse matrix multiplication": the layer is differentiated
 * through its renormalisation, the Hadamard product with A^{l-1}, the softmax
 * and the two sparse products; the kept sets I^l are constants, as top-K is
 * piecewise constant). Gradients of the loss with respect to the forward
 * inputs, given those with respect to its outputs:
 *
 *   G_ij = dA_ij + dO_i . v_j,   g_ij = G_ij - sum_j' A_ij' G_ij'   (j, j' kept)
 *   dQ_i = sum_j A_ij g_ij k_j / sqrt(d)
 *   dK_j = sum_i A_ij g_ij q_i / sqrt(d),   dV_j = sum_i A_ij dO_i
 *   dA_prev_ij = exp(s_ij) / sum_j' A_prev_ij' exp(s_ij') * g_ij at kept slots
 *                (j' kept; = A_ij g_ij / A_prev_ij where A_prev_ij > 0), 0 at
 *                dropped ones; s_ij = q_i.k_j / sqrt(d)
 *
 * Q, K, V, I_prev, A_prev, K_prev, K_l  the forward call's arguments, one index
 *         matrix per head (I_prev NULL = every slot, K_prev = N). Window mode, or
 *         global mode (shape->win = 0, tokens = raster pixels; the individualized
 *         layer of "From Local Windows to Adaptive Candidates via Individualized
 *         Exploratory": a list shared by the heads is passed once per head).
 * I_l, A_l  [B, heads, nwin, N, K_l] the forward call's outputs I^l, A^l.
 *         I_l must be a subsequence of I_prev in I_prev's order (what
 *         pfa_sparse_layer and pfa_dense_layer write).
 * dO      [B, heads, H, W, d] fp32 gradient of O (required).
 * dA_l    [B, heads, nwin, N, K_l] fp32 gradient of A^l (from the next layer's
 *         backward), or NULL for zero.
 * dQ, dK, dV  [B, heads, H, W, d] fp32 outputs, every element written.
 * dA_prev [B, heads, nwin, N, K_prev] fp32 output aligned with I_prev, or NULL
 *         (not computed). Requires A_prev. A kept slot whose A_prev is 0 (kept
 *         when K_l exceeds the row's positive weights) gets the formula's value.
 * workspace  device buffer of at least pfa_sparse_layer_backward_workspace()
 *         bytes (one fp32 per kept pair and one int32 per query row), owned by
 *         the caller; its contents on entry do not matter and are overwritten.
 * The backward pass is deterministic: dK and dV are summed in a fixed order
 * (by row, whatever the scheduling).
 * Errors: PFA_ERR_INVALID for NULL required pointers, inconsistent sizes,
 * dA_prev without A_prev, a workspace that is too small; PFA_ERR_UNSUPPORTED
 * for K_l > 256, global mode with more than 2^22 tokens (8192 with dA_prev),
 * and the shape limits of pfa_sparse_layer.
 */
int pfa_sparse_layer_backward(const pfa_shape* shape, const void* Q, const void* K, const void* V,
                              const int32_t* I_prev, const float* A_prev, int32_t K_prev, int32_t K_l,
                              const int32_t* I_l, const float* A_l, const float* dO, const float* dA_l,
                              float* dQ, float* dK, float* dV, float* dA_prev, void* workspace,
                              int64_t workspace_bytes, void* stream);

/* Workspace bytes pfa_sparse_layer_backward needs for this shape and K_l, or a
 * negative error code (PFA_ERR_INVALID / PFA_ERR_UNSUPPORTED as for the shape,
 * PFA_ERR_INVALID for K_l outside [1, N]). Host only, no device work. */
int64_t pfa_sparse_layer_backward_workspace(const pfa_shape* shape, int32_t K_l);

/*
 * Backward pass of a sparse layer computed with a relative position bias
 * (pfa_sparse_layer_rpb; the bias table is the score term of "Progressive Focused
 * Transformer", which the notes describe as relative position bias based). The
 * bias enters s_ij only, so dQ, dK, dV and dA_prev are those of
 * pfa_sparse_layer_backward (s_ij includes the bias where dA_prev needs the
 * scores), and the bias gradient is the sum of the score gradients over every kept
 * pair of the head with the table entry's offset, across images and windows:
 *   dbias[h][rel(i, j)] = sum over (b, window, i, kept j) of A_ij g_ij.
 *
 * bias    [heads, (2 win - 1)^2] fp32 device table of the forward call, or NULL.
 * dbias   [heads, (2 win - 1)^2] fp32 output (every element written), or NULL (not
 *         computed). Requires bias.
 * workspace  at least pfa_sparse_layer_backward_rpb_workspace() bytes (that of
 *         pfa_sparse_layer_backward, then one table per window-head).
 * Other arguments as pfa_sparse_layer_backward. dbias is summed in a fixed order
 * (no atomics): the same on every run.
 * Errors: as pfa_sparse_layer_backward, PFA_ERR_INVALID for dbias without bias,
 * PFA_ERR_UNSUPPORTED for a bias in global mode.
 */
int pfa_sparse_layer_backward_rpb(const pfa_shape* shape, const void* Q, const void* K, const void* V,
                                  const float* bias, const int32_t* I_prev, const float* A_prev, int32_t K_prev,
                                  int32_t K_l, const int32_t* I_l, const float* A_l, const float* dO,
                                  const float* dA_l, float* dQ, float* dK, float* dV, float* dA_prev, float* dbias,
                                  void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes pfa_sparse_layer_backward_rpb needs (with dbias), or a negative
 * error code as pfa_sparse_layer_backward_workspace (and PFA_ERR_UNSUPPORTED for
 * global mode). Host only. */
int64_t pfa_sparse_layer_backward_rpb_workspace(const pfa_shape* shape, int32_t K_l);

/*
 * Backward pass of the dense first layer (window mode): softmax attention over
 * the window's N slots, P_ij = exp(s_ij - lse_i), O = P V ("Progressive focused
 * resource allocation strategy": the first layer keeps every slot). Its map
 * A^1 = P also feeds the second layer, so dA (the second layer's dA_prev, with
 * I_prev = NULL) is an input besides dO:
 *   G_ij = dA_ij + dO_i . v_j,   D_i = sum_j P_ij G_ij,   dS_ij = P_ij (G_ij - D_i)
 *   dQ = dS K / sqrt(d),   dK = dS^T Q / sqrt(d),   dV = P^T dO.
 *
 * Q, K, V, bias  the forward call's inputs (bias: as pfa_dense_layer_rpb, or NULL).
 * lse     [B, heads, nwin, N] fp32: the forward's lse_out (P is recomputed).
 * dO      [B, heads, H, W, d] fp32 gradient of O.
 * dA      [B, heads, nwin, N, N] fp32 gradient of A^1, or NULL (zero).
 * dQ, dK, dV  [B, heads, H, W, d] fp32 outputs, every element written.
 * workspace  at least pfa_dense_layer_backward_workspace() bytes (one fp32
 *         per query slot), owned by the caller.
 * Deterministic (no atomics). Window sides that are multiples of 8 (of 16 with
 * a bias). Errors: PFA_ERR_INVALID for NULL required pointers or a small
 * workspace; PFA_ERR_UNSUPPORTED for global mode, win % 8 != 0, a bias with
 * win % 16 != 0, and the shape limits of pfa_dense_layer.
 */
int pfa_dense_layer_backward(const pfa_shape* shape, const void* Q, const void* K, const void* V, const float* bias,
                             const float* lse, const float* dO, const float* dA, float* dQ, float* dK, float* dV,
                             void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes pfa_dense_layer_backward needs, or a negative shape error. Host only. */
int64_t pfa_dense_layer_backward_workspace(const pfa_shape* shape);

/*
 * pfa_dense_layer_backward with the gradient of the relative position bias table
 * (see pfa_sparse_layer_backward_rpb): dS_ij = P_ij (G_ij - D_i) summed over every
 * pair of the head with the entry's offset, across images and windows,
 *   dbias[h][rel(i, j)] = sum over (b, window, i, j) of dS_ij.
 *
 * dbias   [heads, (2 win - 1)^2] fp32 output (every element written), or NULL
 *         (then the call is pfa_dense_layer_backward). Requires bias.
 * workspace  at least pfa_dense_layer_backward_rpb_workspace() bytes: one fp32 per
 *         query slot, then, with dbias, 4 win KiB per 16 query slots (per key row
 *         and 16-query block, the sums per column offset) and one table per
 *         window-head.
 * Other arguments, limits and errors as pfa_dense_layer_backward, and
 * PFA_ERR_INVALID for dbias without bias. Deterministic: every sum of dbias runs
 * in a fixed order.
 */
int pfa_dense_layer_backward_rpb(const pfa_shape* shape, const void* Q, const void* K, const void* V,
                                 const float* bias, const float* lse, const float* dO, const float* dA, float* dQ,
                                 float* dK, float* dV, float* dbias, void* workspace, int64_t workspace_bytes,
                                 void* stream);

/* Workspace bytes pfa_dense_layer_backward_rpb needs with dbias, or a negative
 * shape error (PFA_ERR_UNSUPPORTED for global mode). Host only. */
int64_t pfa_dense_layer_backward_rpb_workspace(const pfa_shape* shape);

/*
 * pfa_dense_layer_backward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving or training
 * loops, harnesses that forbid hipMalloc. It computes exactly what
 * pfa_dense_layer_backward computes (the same kernels) and allocates nothing: its
 * scratch memory (one fp32 per query slot) is a static device array of
 * PFA_STATIC_SCRATCH_BYTES in the library's code object. Each GPU the library
 * runs on holds its own copy until the process ends; the first call on a device
 * looks up that copy's address (hipGetSymbolAddress), later calls reuse it.
 *
 * Arguments, layouts, outputs and the other errors are those of
 * pfa_dense_layer_backward. PFA_ERR_TOO_LARGE: more than
 * PFA_STATIC_SCRATCH_BYTES / 4 query slots; nothing is enqueued.
 * Every call on one GPU shares that GPU's array, and each call writes the part it
 * reads before reading it, so calls in order on one stream are safe; calls that
 * overlap on one GPU (on different streams, or from several host threads
 * without ordering) race on the array and may return wrong gradients.
 */
int pfa_dense_layer_backward_noalloc(const pfa_shape* shape, const void* Q, const void* K, const void* V,
                                     const float* bias, const float* lse, const float* dO, const float* dA,
                                     float* dQ, float* dK, float* dV, void* stream);

/*
 * Propagation and sparsification of an individualized index matrix between
 * attention blocks ("From Local Windows to Adaptive Candidates via
 * Individualized Exploratory": propagation and sparsification paragraphs,
 * architecture paragraph with k1 = [22, 20, 14, 12], k2 = [12, 10, 7, 6]).
 * Each token's candidates are pruned to the most similar ones and extended by
 * the neighbours of its neighbours, duplicates removed. With T_k(i) = the k
 * candidates of row i with the largest score (score = the n_maps maps added in
 * fp32 in map order; equal scores keep the lower token index):
 *     I_out(i) = Dedup( T_k1(i)  U  union over u in T_k2(i) of T_k2(u) ).
 *
 * I       [B, N, k] int32 token indices in [0, N), distinct within a row
 *         (global mode: token = raster index of the map).
 * A       [B, n_maps, N, k] fp32 attention weights aligned with I (e.g. the
 *         heads' maps of the block's last layer; finite).
 * I_out   [B, N, k1 + k2*k2] int32: each row's set in ascending order, then -1.
 * count_out [B, N] int32: the set sizes.
 * workspace  at least pfa_iet_propagate_workspace(B, N, k1, k2) bytes of
 *         device memory (the rows' T_k1 and T_k2), owned by the caller.
 * The result is exact (integer), the same on every run.
 * Errors: PFA_ERR_INVALID for sizes < 1, k2 > k1, k1 > k, NULL pointers, a
 * small workspace; PFA_ERR_UNSUPPORTED for k > 64 or N > 65536.
 */
int pfa_iet_propagate(int32_t B, int32_t N, int32_t k, int32_t n_maps, const int32_t* I, const float* A,
                      int32_t k1, int32_t k2, int32_t* I_out, int32_t* count_out, void* workspace,
                      int64_t workspace_bytes, void* stream);

/* Workspace bytes pfa_iet_propagate needs, or PFA_ERR_INVALID for sizes < 1.
 * Host only. */
int64_t pfa_iet_propagate_workspace(int32_t B, int32_t N, int32_t k1, int32_t k2);

/* Static string for a return code; never NULL. */
const char* pfa_strerror(int code);

/* Library version, major*10000 + minor*100 + patch. */
int pfa_version(void);

/*
 * Kernel timing (instrumentation; off by default). While enabled, every kernel
 * the two layer calls enqueue is bracketed by a pair of HIP events recorded on
 * the stream it is launched on, so that a caller can attribute device time to
 * the individual kernels of a layer (a sparse layer may run a selection kernel
 * followed by an aggregation kernel). Not thread-safe: one host thread drives
 * the layer calls while timing is on.
 */
typedef enum {
    PFA_KERNEL_DENSE = 0,          /* dense first layer, all N candidates, MFMA */
    PFA_KERNEL_ALL_CANDIDATES = 1, /* sparse layer whose candidate list is every slot (MFMA scores) */
    PFA_KERNEL_SPARSE = 2,         /* global mode: selection and aggregation in one kernel */
    PFA_KERNEL_SELECT = 3,         /* window mode: selection only (I^l, A^l) */
    PFA_KERNEL_AGGREGATE = 4,      /* window mode: O from the stored (I^l, A^l) rows */
    PFA_KERNEL_IOTA = 5,           /* I rows 0..N-1 of the dense layer */
    PFA_KERNEL_BWD_ROWS = 6,       /* backward: per-row pass(es) -> g, dQ, dA_prev */
    PFA_KERNEL_BWD_SCATTER = 7,    /* backward: dK, dV per window-head ("bwd_dkv_kernel" on MFMA, or
                                      "bwd_dkv_sorted_kernel" from the kept pairs sorted by token) */
    PFA_KERNEL_IET_RANK = 8,       /* index propagation: top-k1 / top-k2 of each row */
    PFA_KERNEL_IET_UNION = 9,      /* index propagation: de-duplicated union per row */
    PFA_KERNEL_DENSE_BWD = 10,     /* backward of the dense layer ("dense_bwd_dq_kernel" then
                                      "dense_bwd_dkv_kernel", one record for both) */
    PFA_KERNEL_BWD_EXACT = 11,     /* backward with dA_prev: rows whose kept weights include zero or
                                      subnormal values, dA_prev from the scores */
    PFA_KERNEL_DBIAS = 12,         /* backward with a bias gradient: per window-head tables
                                      ("dbias_sparse_wh_kernel" or "dbias_dense_fold_kernel") then
                                      "dbias_reduce_kernel", one record for both */
    PFA_KERNEL_FIRST_MAP = 13      /* backward of the fused first two layers: the first layer's map at
                                      the second layer's kept slots ("first_map_kept_kernel"), and its
                                      gradient spread into dense rows ("spread_rows_kernel") */
} pfa_kernel_kind;

/* capacity > 0: create 2*capacity events and start recording (earlier records
 * are discarded); capacity == 0: stop and destroy the events. Launches past the
 * capacity run untimed and are counted as dropped. Errors: PFA_ERR_INVALID for
 * capacity < 0 or > 2^20; PFA_ERR_HIP if event creation fails (timing stays off). */
int pfa_timing_enable(int32_t capacity);

/* Number of launches recorded since the last read (no synchronisation). */
int32_t pfa_timing_count(void);

/* Wait for the recorded events and copy up to `cap` records, in launch order:
 * kinds[i] (pfa_kernel_kind) and ms[i] (elapsed milliseconds between the two
 * events around launch i). *n_out = records copied; *dropped (may be NULL) =
 * launches not returned (past the capacity or past `cap`). The record list is
 * then cleared. kinds/ms are host arrays owned by the caller.
 * Errors: PFA_ERR_INVALID for NULL n_out, cap < 0, NULL arrays with cap > 0;
 * PFA_ERR_HIP if an event query fails. */
int pfa_timing_read(int32_t* kinds, float* ms, int32_t cap, int32_t* n_out, int32_t* dropped);

/* Family name of a pfa_kernel_kind: profilers show the family's kernel symbols
 * beginning with it ("sparse_layer_kernel(select)" names the selection-only
 * instantiations of sparse_layer_kernel); "unknown" for other values. Never NULL. */
const char* pfa_kernel_name(int32_t kind);

#ifdef __cplusplus
}
#endif

#endif /* PFA_H */
