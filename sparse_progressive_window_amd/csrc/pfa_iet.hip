// Propagation and sparsification of an individualized index matrix on gfx950.
//
// "From Local Windows to Adaptive Candidates via Individualized Exploratory"
// (propagation and sparsification paragraphs, architecture paragraph): between
// attention blocks, each token's candidates are pruned to the most similar ones
// and extended by the neighbours of its neighbours, duplicates removed. With
// T_k(i) = the k candidates of row i with the largest score (the heads' maps
// added in fp32 in head order; ties to the lower token index), the new set is
//   Dedup( T_k1(i)  U  union over u in T_k2(i) of T_k2(u) ).
//
// iet_rank_kernel: one wavefront per row, lane c holds candidate c (k <= 64);
//   its rank is the number of candidates that beat it, counted over the row's
//   lanes read back one at a time (v_readlane); ranks < k1 / < k2 write T1 / T2
//   (the workspace), in rank order.
// iet_union_kernel: one wavefront per row marks the k1 + k2^2 tokens in an LDS
//   bitmap of the N tokens, then reads the bitmap in word order: a wavefront
//   prefix sum of the words' popcounts places every set bit, so the output row
//   is ascending without a sort; the rest of the row is padded with -1.
#include <limits.h>

#include "pfa_kernels.h"

namespace pfa {
namespace {

constexpr int kIetWaves = 4;

__device__ __forceinline__ int read_lane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float read_lane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__global__ __launch_bounds__(kIetWaves * kWave) void iet_rank_kernel(const IetArgs p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * kIetWaves + threadIdx.x / kWave;
    const int64_t rows = (int64_t)p.B * p.N;
    if (row >= rows) return;                       // whole wavefront
    const int64_t b = row / p.N;
    const int64_t i = row - b * p.N;
    const int k = p.k;
    float sc = -INFINITY;
    int j = INT_MAX;
    if (lane < k) {
        j = p.I[row * k + lane];
        sc = 0.0f;
        for (int h = 0; h < p.n_maps; ++h) sc += p.A[((b * p.n_maps + h) * p.N + i) * k + lane];
    }
    int rank = 0;
    for (int c = 0; c < k; ++c) {
        const float so = read_lane_f(sc, c);
        const int jo = read_lane_i(j, c);
        rank += (so > sc || (so == sc && jo < j)) ? 1 : 0;
    }
    if (lane < k) {
        if (rank < p.k1) p.T1[row * p.k1 + rank] = j;
        if (rank < p.k2) p.T2[row * p.k2 + rank] = j;
    }
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_up(x, o);
        if (lane >= o) x += t;
    }
    return x;
}

__global__ __launch_bounds__(kIetWaves * kWave) void iet_union_kernel(const IetArgs p) {
    extern __shared__ uint32_t bitmaps[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t row = (int64_t)blockIdx.x * kIetWaves + wave;
    const int64_t rows = (int64_t)p.B * p.N;
    if (row >= rows) return;                       // whole wavefront; no workgroup barrier below
    const int N = p.N;
    const int nw = (N + 31) >> 5;
    uint32_t* bm = bitmaps + wave * nw;
    for (int w = lane; w < nw; w += kWave) bm[w] = 0u;
    const int64_t b = row / N;
    const int k1 = p.k1, k2 = p.k2;
    const int32_t* t1 = p.T1 + row * k1;
    const int32_t* t2 = p.T2 + row * k2;
    const int32_t* t2b = p.T2 + b * N * k2;        // T2 rows of this image
    // token values are clamped into [0, N) for memory safety only (precondition)
    for (int c = lane; c < k1; c += kWave) {
        const int v = (int)min((unsigned)t1[c], (unsigned)(N - 1));
        atomicOr(&bm[v >> 5], 1u << (v & 31));
    }
    for (int e = lane; e < k2 * k2; e += kWave) {
        const int q = e / k2;
        const int u = (int)min((unsigned)t2[q], (unsigned)(N - 1));
        const int v = (int)min((unsigned)t2b[(int64_t)u * k2 + (e - q * k2)], (unsigned)(N - 1));
        atomicOr(&bm[v >> 5], 1u << (v & 31));
    }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int width = k1 + k2 * k2;
    int32_t* out = p.I_out + row * width;
    int base = 0;
    for (int w0 = 0; w0 < nw; w0 += kWave) {
        const int w = w0 + lane;
        uint32_t bits = w < nw ? bm[w] : 0u;
        const int cnt = __builtin_popcount(bits);
        const int incl = wave_incl_scan(cnt, lane);
        int pos = base + incl - cnt;
        while (bits) {
            const int bit = __builtin_ctz(bits);
            if (pos < width) out[pos] = w * 32 + bit;
            ++pos;
            bits &= bits - 1u;
        }
        base += read_lane_i(incl, kWave - 1);
    }
    for (int c = base + lane; c < width; c += kWave) out[c] = -1;
    if (lane == 0) p.count_out[row] = min(base, width);
}

}  // namespace

int iet_union_lds(int N) { return kIetWaves * ((N + 31) / 32) * 4; }

hipError_t launch_iet_rank(const IetArgs& a, hipStream_t s) {
    const int64_t rows = (int64_t)a.B * a.N;
    const int64_t grid = (rows + kIetWaves - 1) / kIetWaves;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(iet_rank_kernel, dim3((unsigned)grid), dim3(kIetWaves * kWave), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_iet_union(const IetArgs& a, hipStream_t s) {
    const int64_t rows = (int64_t)a.B * a.N;
    const int64_t grid = (rows + kIetWaves - 1) / kIetWaves;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    const int lds = iet_union_lds(a.N);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(iet_union_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(iet_union_kernel, dim3((unsigned)grid), dim3(kIetWaves * kWave), lds, s, a);
    return hipGetLastError();
}

}  // namespace pfa
