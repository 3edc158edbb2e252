// Gradient of the relative position bias table on gfx950.
//
// With a bias ("Progressive Focused Transformer" notes: the network is relative
// position bias based) the score is s_ij = q_i.k_j / sqrt(d) + bias[h][rel(i, j)],
// rel(i, j) = (iy - jy + win - 1)(2 win - 1) + (ix - jx + win - 1) for the
// window-local slots i = (iy, ix), j = (jy, jx). The table entry enters each score
// of its offset once, so its gradient is the sum of the score gradients dS_ij over
// every pair of the head with that offset, across images and windows:
//   dbias[h][r] = sum over (b, window, i, j) with rel(i, j) = r of dS_ij,
// dS_ij = A_ij g_ij at the kept pairs of a sparse layer (zero at the others), and
// P_ij (G_ij - D_i) over all pairs of the dense layer.
//
// Every sum runs in a fixed order (no floating-point atomics): dbias is the same on
// every run.
// * dbias_sparse_wh_kernel: one workgroup per window-head, 4 wavefronts, each with
//   its own LDS table. A wavefront takes its rows in order; the kept tokens of a row
//   are distinct, so are its offsets, and one wavefront's LDS accesses complete in
//   issue order, so plain read-add-write updates are exact. The four tables are then
//   added in wave order.
// * dbias_dense_fold_kernel: the dense layer's dQ kernel leaves, per wavefront of 16
//   queries (one window row) and per key row, the dS sums of each column offset;
//   one workgroup per window-head adds them up per offset, rows in order.
// * dbias_reduce_kernel: per head and offset, the window-head tables over images and
//   windows in order.
#include "pfa_kernels.h"

namespace pfa {
namespace {

constexpr int kDbiasWaves = 4;
constexpr int kDbiasRows = 4;   // rows whose loads are in flight together per wavefront

// entries per lane of a kept row: EPL = ceil(K_l / 64)
template <int EPL>
__global__ __launch_bounds__(kDbiasWaves * kWave) void dbias_sparse_wh_kernel(const DbiasArgs p) {
    extern __shared__ float tab[];   // [kDbiasWaves][nrel]
    const Geom g = p.g;
    const int win = g.win;
    const int wrow = 2 * win - 1;
    const int nrel = wrow * wrow;
    const int N = g.N;
    const int K_l = p.K_l;
    const int wh = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    for (int u = threadIdx.x; u < kDbiasWaves * nrel; u += blockDim.x) tab[u] = 0.0f;
    __syncthreads();
    float* T = tab + wave * nrel;
    const size_t base = (size_t)wh * N * K_l;
    const int32_t* Ih = p.I_l + base;
    const float* Ah = p.A_l + base;
    const float* Gh = p.g_buf + base;

    struct Batch {
        int j[kDbiasRows][EPL];
        float v[kDbiasRows][EPL];
    };
    // rows i0 + kDbiasWaves r (r < kDbiasRows) of this wavefront
    auto load = [&](Batch& b, int i0) {
#pragma unroll
        for (int r = 0; r < kDbiasRows; ++r) {
            const int i = i0 + kDbiasWaves * r;
#pragma unroll
            for (int x = 0; x < EPL; ++x) {
                const int e = lane + kWave * x;
                const bool ok = i < N && e < K_l;
                const size_t o = ok ? (size_t)i * K_l + e : 0;
                b.j[r][x] = ok ? (int)min((unsigned)Ih[o], (unsigned)(N - 1)) : -1;
                b.v[r][x] = ok ? Ah[o] * Gh[o] : 0.0f;
            }
        }
    };
    const int step = kDbiasWaves * kDbiasRows;
    Batch cur;
    load(cur, wave);
    for (int i0 = wave; i0 < N; i0 += step) {
        Batch nxt;
        if (i0 + step < N) load(nxt, i0 + step);
#pragma unroll
        for (int r = 0; r < kDbiasRows; ++r) {
            const int i = i0 + kDbiasWaves * r;
            const int iy = i / win;
            const int ibase = (iy + win - 1) * wrow + (i - iy * win) + win - 1;
#pragma unroll
            for (int x = 0; x < EPL; ++x) {
                const int j = cur.j[r][x];
                if (j >= 0) {
                    const int jy = j / win;
                    T[ibase - jy * wrow - (j - jy * win)] += cur.v[r][x];
                }
            }
        }
        cur = nxt;
    }
    __syncthreads();
    float* out = p.part + (size_t)wh * nrel;
    for (int u = threadIdx.x; u < nrel; u += blockDim.x) {
        float s = tab[u];
#pragma unroll
        for (int w = 1; w < kDbiasWaves; ++w) s += tab[w * nrel + u];
        out[u] = s;
    }
}

// rows: [wh][N / 16 waves][win key rows][64 lanes]; wave v holds queries 16 v ..
// 16 v + 15 (window row v / (win / 16)) and lane L the column offset L - (win - 1)
__global__ __launch_bounds__(256) void dbias_dense_fold_kernel(const DbiasArgs p) {
    const Geom g = p.g;
    const int win = g.win;
    const int wrow = 2 * win - 1;
    const int nrel = wrow * wrow;
    const int wpq = win / 16;    // waves per window row of queries
    const int nwv = g.N / 16;
    const int wh = blockIdx.x;
    const float* R = p.rows + (size_t)wh * nwv * win * 64;
    for (int u = threadIdx.x; u < nrel; u += blockDim.x) {
        const int dyi = u / wrow;
        const int col = u - dyi * wrow;
        const int dy = dyi - (win - 1);     // query row - key row
        const int qa = dy > 0 ? dy : 0;
        const int qb = dy < 0 ? win - 1 + dy : win - 1;
        float s = 0.0f;
        for (int qy = qa; qy <= qb; ++qy) {
            const int ky = qy - dy;
            for (int x = 0; x < wpq; ++x) s += R[((size_t)(qy * wpq + x) * win + ky) * 64 + col];
        }
        p.part[(size_t)wh * nrel + u] = s;
    }
}

__global__ __launch_bounds__(256) void dbias_reduce_kernel(const DbiasArgs p) {
    const Geom g = p.g;
    const int wrow = 2 * g.win - 1;
    const int nrel = wrow * wrow;
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= g.heads * nrel) return;
    const int h = idx / nrel;
    const int u = idx - h * nrel;
    const int nwin = g.nwy * g.nwx;
    float s = 0.0f;
    for (int b = 0; b < g.B; ++b) {
        const float* src = p.part + ((size_t)(b * g.heads + h) * nwin) * nrel + u;
        for (int w = 0; w < nwin; ++w) s += src[(size_t)w * nrel];
    }
    p.dbias[idx] = s;
}

hipError_t launch_reduce(const DbiasArgs& a, hipStream_t s) {
    const int wrow = 2 * a.g.win - 1;
    const int total = a.g.heads * wrow * wrow;
    hipLaunchKernelGGL(dbias_reduce_kernel, dim3((total + 255) / 256), dim3(256), 0, s, a);
    return hipGetLastError();
}

int64_t n_wh_of(const Geom& g) { return (int64_t)g.B * g.heads * g.nwy * g.nwx; }

}  // namespace

int dbias_sparse_lds(int win) { return kDbiasWaves * (2 * win - 1) * (2 * win - 1) * 4; }

hipError_t launch_dbias_sparse(const DbiasArgs& a, hipStream_t s) {
    const int lds = dbias_sparse_lds(a.g.win);
    const int grid = (int)n_wh_of(a.g);
    const void* fn = a.K_l <= kWave       ? reinterpret_cast<const void*>(dbias_sparse_wh_kernel<1>)
                     : a.K_l <= 2 * kWave ? reinterpret_cast<const void*>(dbias_sparse_wh_kernel<2>)
                                          : reinterpret_cast<const void*>(dbias_sparse_wh_kernel<4>);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    if (a.K_l <= kWave)
        hipLaunchKernelGGL(dbias_sparse_wh_kernel<1>, dim3(grid), dim3(kDbiasWaves * kWave), lds, s, a);
    else if (a.K_l <= 2 * kWave)
        hipLaunchKernelGGL(dbias_sparse_wh_kernel<2>, dim3(grid), dim3(kDbiasWaves * kWave), lds, s, a);
    else
        hipLaunchKernelGGL(dbias_sparse_wh_kernel<4>, dim3(grid), dim3(kDbiasWaves * kWave), lds, s, a);
    e = hipGetLastError();
    return e == hipSuccess ? launch_reduce(a, s) : e;
}

hipError_t launch_dbias_dense(const DbiasArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(dbias_dense_fold_kernel, dim3((int)n_wh_of(a.g)), dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? launch_reduce(a, s) : e;
}

}  // namespace pfa
