// Backward of the first two layers computed together (pfa_first_two_layers).
//
// The fused forward never writes the first layer's map A^1 = P (paper notes
// "Progressive Focused Transformer for Single Image Super-Resolution", sections
// "Progressive attention across layers" and "Progressive focused resource
// allocation strategy": layer 1 keeps every slot, layer 2 selects from A^1). The
// second layer's backward reads A^1 only at its kept slots (dA^1 = dkey / A^1 there,
// and the exact form's normaliser), and gives dA^1 = 0 at the dropped ones. So the
// second layer's backward runs with its own kept set as the candidate list (the
// same gradients: the dropped slots' terms are zero) on A^1 recomputed at those
// slots only, from q1, k1 and the first layer's log denominators:
//   A^1_ij = exp(s1_ij - lse1_i),  s1_ij = q1_i.k1_j / sqrt(d),
// and its dA^1 rows (aligned with I^2) are spread into the dense [N, N] rows that
// the first layer's backward reads.
//
// first_map_kept_kernel: 16 wavefronts per workgroup of 512 rows, the window's k1
// rows staged in LDS; a wavefront takes a row, its lanes the row's kept slots. Each
// lane reads the 16-byte chunks of its k1 row (and of the query) in a lane-rotated
// order, so the gathers of random rows spread over the LDS banks; bf16 products
// are taken on the packed pairs (v_dot2c_f32_bf16: exact products, fp32 sums).
// A^1 is written aligned with I^2 (coalesced).
// spread_rows_kernel: one wavefront per row: the dense row is built in the wave's
// LDS row (zeros, then the K2 values at their slots; one wave's LDS accesses
// complete in issue order) and written out in 16-byte stores.
#include "pfa_kernels.h"
#include "pfa_rows.h"

namespace pfa {
namespace {

constexpr int kMapWaves = 16;
constexpr int kMapRows = 512;   // rows per workgroup
constexpr float kLog2eF = 1.4426950408889634f;

template <typename T, int D>
__global__ __launch_bounds__(kMapWaves * kWave) void first_map_kept_kernel(const FirstMapArgs p) {
    constexpr int EPC = Chunk<T>::kElems;
    constexpr int CH = D / EPC;
    constexpr int ROWB = D * (int)sizeof(T);
    extern __shared__ __align__(16) unsigned char smem[];
    const Geom g = p.g;
    const int N = g.N;
    const int K2 = p.K2;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const WhPart w = decode_block(p.blocks_per_wh, p.xcd_map, g);
    const size_t plane = (size_t)w.bh * g.H * g.W * D;
    stage_rows<T, D>(smem, ROWB, static_cast<const T*>(p.K1) + plane, g, w.wy, w.wx);
    __syncthreads();
    const int row0 = w.part * kMapRows;
    const int row1 = min(N, row0 + kMapRows);
    const T* Qh = static_cast<const T*>(p.Q1) + plane;
    constexpr int MAXU = 4;   // kept slots per lane (the caller admits K2 <= 256)
    int coff[CH];   // lane-rotated chunk order
#pragma unroll
    for (int m = 0; m < CH; ++m) coff[m] = ((m + lane) % CH) * 16;
    const int nu = (K2 + kWave - 1) / kWave;
    for (int i = row0 + wave; i < row1; i += kMapWaves) {
        const size_t row = (size_t)w.wh * N + i;
        const int32_t* Ir = p.I2 + row * K2;
        float* Ar = p.A1 + row * K2;
        // the row's kept slots first, then the query chunks: their loads overlap
        int jv[MAXU];
#pragma unroll
        for (int u = 0; u < MAXU; ++u) {
            const int e = lane + kWave * u;
            jv[u] = (u < nu && e < K2) ? (int)min((unsigned)Ir[e], (unsigned)(N - 1)) : 0;
        }
        const unsigned char* qr = reinterpret_cast<const unsigned char*>(Qh + (size_t)slot_pixel(g, w.wy, w.wx, i) * D);
        uint4 qc[CH];
#pragma unroll
        for (int m = 0; m < CH; ++m) qc[m] = *reinterpret_cast<const uint4*>(qr + coff[m]);
        const float l2 = p.lse1[row] * kLog2eF;
#pragma unroll
        for (int u = 0; u < MAXU; ++u) {
            if (u >= nu) break;   // uniform
            const int e = lane + kWave * u;
            const unsigned char* kr = smem + jv[u] * ROWB;
            float acc = 0.0f;
#pragma unroll
            for (int m = 0; m < CH; ++m) {
                const uint4 kc = *reinterpret_cast<const uint4*>(kr + coff[m]);
                if constexpr (sizeof(T) == 2) {
                    acc = dot2_bf16(qc[m].x, kc.x, acc);
                    acc = dot2_bf16(qc[m].y, kc.y, acc);
                    acc = dot2_bf16(qc[m].z, kc.z, acc);
                    acc = dot2_bf16(qc[m].w, kc.w, acc);
                } else {
                    acc = fmaf(__uint_as_float(qc[m].x), __uint_as_float(kc.x), acc);
                    acc = fmaf(__uint_as_float(qc[m].y), __uint_as_float(kc.y), acc);
                    acc = fmaf(__uint_as_float(qc[m].z), __uint_as_float(kc.z), acc);
                    acc = fmaf(__uint_as_float(qc[m].w), __uint_as_float(kc.w), acc);
                }
            }
            if (e < K2) Ar[e] = fast_exp2(fmaf(acc, p.scale2, -l2));
        }
    }
}

constexpr int kSpreadWaves = 4;

// dense[row][0..N) = 0, then dense[row][I[row][e]] = vals[row][e] (N <= 1024, a multiple of 4)
__global__ __launch_bounds__(kSpreadWaves * kWave) void spread_rows_kernel(const SpreadArgs p) {
    __shared__ __align__(16) float rowbuf[kSpreadWaves][1024];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    float* rb = rowbuf[wave];
    const int N = p.N, K = p.K;
    const int64_t row = (int64_t)blockIdx.x * kSpreadWaves + wave;
    if (row >= p.rows) return;
    for (int x = lane * 4; x < N; x += 4 * kWave) *reinterpret_cast<float4*>(rb + x) = make_float4(0.f, 0.f, 0.f, 0.f);
    const int32_t* Ir = p.I + row * K;
    const float* vr = p.vals + row * K;
    for (int e = lane; e < K; e += kWave) rb[min((unsigned)Ir[e], (unsigned)(N - 1))] = vr[e];
    float* out = p.dense + row * N;
    for (int x = lane * 4; x < N; x += 4 * kWave) *reinterpret_cast<float4*>(out + x) = *reinterpret_cast<const float4*>(rb + x);
}

template <typename T, int D>
hipError_t launch_map_t(const FirstMapArgs& a, int grid, hipStream_t s) {
    const int lds = a.g.N * D * (int)sizeof(T);
    const void* fn = reinterpret_cast<const void*>(first_map_kept_kernel<T, D>);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((first_map_kept_kernel<T, D>), dim3(grid), dim3(kMapWaves * kWave), lds, s, a);
    return hipGetLastError();
}

}  // namespace

int first_map_blocks(int N) { return (N + kMapRows - 1) / kMapRows; }

hipError_t launch_spread_rows(const SpreadArgs& a, hipStream_t stream) {
    if (a.N > 1024 || a.N % 4) return hipErrorInvalidValue;
    const int64_t grid = (a.rows + kSpreadWaves - 1) / kSpreadWaves;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(spread_rows_kernel, dim3((int)grid), dim3(kSpreadWaves * kWave), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_first_map(const FirstMapArgs& a, int dtype, int D, int grid, hipStream_t stream) {
    if (a.g.N * D * (dtype == 0 ? 4 : 2) > kLdsBytes) return hipErrorInvalidValue;
    if (dtype == 0) return D == 16 ? launch_map_t<float, 16>(a, grid, stream) : launch_map_t<float, 32>(a, grid, stream);
    return D == 16 ? launch_map_t<uint16_t, 16>(a, grid, stream) : launch_map_t<uint16_t, 32>(a, grid, stream);
}

}  // namespace pfa
