// Kernel argument blocks and launchers (internal to libpfa.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pfa_device.h"

namespace pfa {

constexpr int kScratchBytes = 32 * 1024;  // per workgroup: (j, weight) entries for the aggregation
constexpr int kLdsBytes = 160 * 1024;     // LDS per workgroup on gfx950

struct SparseArgs {
    const void* Q;
    const void* K;
    const void* V;
    const int32_t* I_prev;   // nullptr: all slots in order
    const float* A_prev;     // nullptr: all ones
    int32_t* I_out;
    float* A_out;
    float* O_out;
    Geom g;
    int K_prev, K_l;
    int i_shared;
    int rows_per_block, blocks_per_wh;
    int xcd_map;             // 1: the parts of a window-head run on one XCD (needs #wh % 8 == 0)
    float scale2;            // log2(e) / sqrt(d): scores are kept in base-2 units
    // fused first two layers only: the first layer's Q and K (window slots under
    // shift1); the candidate scores are then q1.k1 + q.k
    const void* Q1;
    const void* K1;
    int shift1;
    // window mode, selection kernels: the layer's relative position bias, one
    // (2 win - 1)^2 table per head (nullptr: none)
    const float* bias;
};

// kKselect: window mode, K staged in LDS, selection only (O comes from
// launch_aggregate); kKVglobal: global mode, K and V read from global memory,
// selection and aggregation in one kernel.
enum SparseMode { kKVglobal = 0, kKselect = 1 };

struct DenseArgs {
    const void* Q;
    const void* K;
    const void* V;
    float* A_out;            // nullptr: O-only
    float* lse_out;          // nullptr: no log-normaliser output
    float* O_out;
    Geom g;
    float scale2;
    int xcd_map;             // 1: the query blocks of a window-head run on one XCD (needs #wh % 8 == 0)
    const float* bias;       // relative position bias, one (2 win - 1)^2 table per head, or nullptr
};

// Backward pass of a window-mode sparse layer with the kept sets held fixed.
struct BackwardArgs {
    const void* Q;
    const void* K;
    const void* V;
    const int32_t* I_prev;   // nullptr: slot p holds token p (K_prev == N)
    const float* A_prev;     // read only when dA_prev is written
    const int32_t* I_l;      // the layer's kept slots [wh, N, K_l]
    const float* A_l;        // the layer's map [wh, N, K_l]
    const float* dO;         // [B, heads, H, W, d]
    const float* dA_l;       // [wh, N, K_l] or nullptr (zero)
    float* dQ;
    float* dK;
    float* dV;
    float* dA_prev;          // [wh, N, K_prev] or nullptr (not wanted)
    float* g_buf;            // workspace [wh, N, K_l]: G_ij - sum_j A_ij G_ij
    int32_t* row_flags;      // workspace, one int per row-pass workgroup (with dA_prev): 1 where a kept
                             // A^l of its rows is zero or subnormal (those rows need the exact pass)
    Geom g;
    int K_prev, K_l;
    int rows_per_block, blocks_per_wh;
    int xcd_map;
    float scale;             // 1 / sqrt(d)
    float scale2;            // log2(e) / sqrt(d): base-2 scores of the exact dA^{l-1} pass
    const float* bias;       // the forward's relative position bias [heads, (2 win - 1)^2], or nullptr
    // dK/dV MFMA kernel: workgroups [0, dkv_full) take a whole window-head each;
    // each further pair (workgroups 8 apart, one XCD) takes the two token halves
    // of one window-head (balances the last round over the CUs)
    int dkv_full;
    // sorted dK/dV kernel, one matrix per workgroup: (window-head, token range)
    // units; workgroups 8n + x and 8(n + 1) + x (n even) take the dV and the dK of
    // unit 8(n / 2) + x
    int dkv_units;
};

// Row pass: with both K and V staged (when they fit in LDS together), or as a
// V pass (g rows) followed by a K pass (dQ, dA_prev). `parts` = workgroups per
// window-head for the scatter pass.
int backward_fused_rows(int dtype, int D, int N, int K_l, bool want_dA_prev);
hipError_t launch_backward_rows(const BackwardArgs& a, int dtype, int D, bool has_v, bool has_k, int grid,
                                hipStream_t stream);
// dA^{l-1} of the rows the row pass flagged, from the scores (after the row pass).
hipError_t launch_backward_exact_dap(const BackwardArgs& a, int dtype, int D, int grid, hipStream_t stream);
// dK and dV from the kept pairs sorted by token per row chunk (work in proportion
// to K_l). A unit is a window-head and up to 1024 of its tokens; split: two
// workgroups per unit (dV, dK; grid 2 * units rounded up to 16, dkv_units set),
// else one (grid = units).
bool backward_dkv_sorted(int dtype, int D, int N, int K_l);
bool backward_dkv_sorted_split(int dtype, int D, int N, int K_l, int64_t units, int cus);
hipError_t launch_backward_dkv_sorted(const BackwardArgs& a, int dtype, int D, bool split, int grid,
                                      hipStream_t stream);
// dK and dV as dense MFMA products over LDS-densified row blocks (N % 16 == 0).
bool backward_dkv_mfma(int D, int N, int K_l);
// whole-window-head dK/dV workgroups for n_wh window-heads on `cus` compute units
// (n_wh when no split applies); the grid is dkv_full + 2 (n_wh - dkv_full)
int64_t backward_dkv_full(int64_t n_wh, int N, int cus);
hipError_t launch_backward_dkv(const BackwardArgs& a, int dtype, int D, int grid, hipStream_t stream);

// Backward pass of the dense first layer.
struct DenseBwdArgs {
    const void* Q;
    const void* K;
    const void* V;
    const float* bias;       // relative position bias, one (2 win - 1)^2 table per head, or nullptr
    const float* lse;        // [wh, N] the forward's ln sum_j exp(s_ij)
    const float* dO;         // [B, heads, H, W, d]
    const float* dA;         // [wh, N, N] gradient of the map, or nullptr
    float* dQ;
    float* dK;
    float* dV;
    float* Dws;              // workspace [wh, N]: D_i = sum_j P_ij G_ij
    float* dbias_rows;       // workspace [wh, N / 16, win, 64]: per wave and key row, the dS sums per
                             // column offset (lane dx + win - 1), or nullptr (no bias gradient)
    Geom g;
    float scale2;            // log2(e) / sqrt(d)
    float scale;             // 1 / sqrt(d)
    int xcd_map;
};
int dense_bwd_blocks(int N);   // workgroups per window-head (each kernel)
hipError_t launch_dense_backward(const DenseBwdArgs& a, int dtype, int D, int grid, hipStream_t stream);

// Gradient of the relative position bias table: per window-head tables (of a
// sparse layer from its kept pairs, of the dense layer from the dQ kernel's rows),
// then summed over images and windows per head. Fixed summation order throughout.
struct DbiasArgs {
    const int32_t* I_l;      // sparse: kept slots [wh, N, K_l]
    const float* A_l;        // sparse: the layer's map [wh, N, K_l]
    const float* g_buf;      // sparse: g per kept pair [wh, N, K_l] (the row pass's workspace)
    const float* rows;       // dense: DenseBwdArgs::dbias_rows
    float* part;             // workspace [wh, (2 win - 1)^2]: per window-head tables
    float* dbias;            // [heads, (2 win - 1)^2] output
    Geom g;
    int K_l;
};
hipError_t launch_dbias_sparse(const DbiasArgs& a, hipStream_t stream);
hipError_t launch_dbias_dense(const DbiasArgs& a, hipStream_t stream);
int dbias_sparse_lds(int win);

// Backward of the fused first two layers: the first layer's map at the second
// layer's kept slots, recomputed into a dense-layout buffer.
struct FirstMapArgs {
    const void* Q1;
    const void* K1;
    const int32_t* I2;       // [wh, N, K2] the second layer's kept slots
    const float* lse1;       // [wh, N] the first layer's log denominators
    float* A1;               // [wh, N, K2] A^1 at the kept slots, aligned with I2
    Geom g;                  // the first layer's geometry (its shift)
    int K2;
    float scale2;            // log2(e) / sqrt(d)
    int blocks_per_wh, xcd_map;
};
int first_map_blocks(int N);
hipError_t launch_first_map(const FirstMapArgs& a, int dtype, int D, int grid, hipStream_t stream);
// dense [rows, N] rows from [rows, K] values at the slots I (zeros elsewhere)
struct SpreadArgs {
    const int32_t* I;
    const float* vals;
    float* dense;
    int64_t rows;
    int N, K;
};
hipError_t launch_spread_rows(const SpreadArgs& a, hipStream_t stream);

// Propagation / sparsification of an individualized index matrix.
struct IetArgs {
    const int32_t* I;        // [B, N, k] token indices
    const float* A;          // [B, n_maps, N, k] maps aligned with I
    int32_t* I_out;          // [B, N, k1 + k2*k2] ascending, -1 padded
    int32_t* count_out;      // [B, N]
    int32_t* T1;             // workspace [B, N, k1]: top-k1 tokens of each row
    int32_t* T2;             // workspace [B, N, k2]
    int B, N, k, n_maps, k1, k2;
};
int iet_union_lds(int N);
hipError_t launch_iet_rank(const IetArgs& a, hipStream_t stream);
hipError_t launch_iet_union(const IetArgs& a, hipStream_t stream);

hipError_t launch_sparse(const SparseArgs& a, int dtype, int D, SparseMode mode, int lds_bytes, int grid,
                         hipStream_t stream);
// All-candidates layer (I^{l-1} implicit, K_prev = N = 1024): MFMA scores, selection only.
hipError_t launch_all_cand(const SparseArgs& a, int dtype, int D, int grid, hipStream_t stream);
// Same with the first layer's scores added (fused first two layers, no A^1).
bool all_cand_dual_fits(int dtype, int D);
hipError_t launch_all_cand_dual(const SparseArgs& a, int dtype, int D, int grid, hipStream_t stream);
// O from stored (I^l, A^l) rows with V in LDS (window mode).
hipError_t launch_aggregate(const SparseArgs& a, int dtype, int D, int grid, hipStream_t stream);
int dense_query_blocks(int N);   // workgroups per window-head of the dense layer
hipError_t launch_dense(const DenseArgs& a, int dtype, int D, int grid, hipStream_t stream);
hipError_t launch_iota_rows(int32_t* I, int64_t rows, int N, hipStream_t stream);

}  // namespace pfa
