// Dense first PFA layer on gfx950 matrix cores.
//
// The first layer keeps every token of the window and computes the complete
// softmax map (paper notes "Progressive Focused Transformer for Single Image
// Super-Resolution", section "Progressive focused resource allocation
// strategy"): A^1 = softmax(Q K^T / sqrt(d)) per window-head, O = A^1 V.
//
// One wave owns 16 query rows. Scores are produced transposed, S^T = K Q^T, with
// 16x16 MFMA tiles (16 keys x 16 queries): the accumulator layout then gives each
// lane 4 consecutive keys of one query, which is exactly the A-operand layout of
// the following P.V MFMA, so probabilities never leave registers. The
// contraction index of the score MFMAs is permuted so that every lane reads a
// contiguous run of d/4 elements of its K and Q rows.
//   fp32 inputs: v_mfma_f32_16x16x4_f32 (exact products, fp32 accumulation).
//   bf16 inputs: v_mfma_f32_16x16x16_bf16; P is split into bf16 hi + lo parts
//   (two MFMAs) so the P.V product keeps ~16 bits of P.
// Two passes over the keys: (1) running row max / row sum, (2) recompute the
// scores, write A^1 (optional) and accumulate O.
#include "pfa_kernels.h"

namespace pfa {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));

template <typename T, int D>
struct DenseOps;

// fp32: lane l covers dims [DPL*grp, DPL*grp + DPL) of its row, DPL = D/4, one
// MFMA step (k = 4: one dim per lane group) per dim of the run.
template <int D>
struct DenseOps<float, D> {
    static constexpr int DPL = D / 4;
    struct Row { float v[DPL]; };
    __device__ static Row load(const float* row, int grp) {
        Row r;
        const float* src = row + grp * DPL;
#pragma unroll
        for (int x = 0; x < DPL; x += 4) {
            const float4 f = *reinterpret_cast<const float4*>(src + x);
            r.v[x] = f.x; r.v[x + 1] = f.y; r.v[x + 2] = f.z; r.v[x + 3] = f.w;
        }
        return r;
    }
    __device__ static v4f scores(const Row& k, const Row& q) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int x = 0; x < DPL; ++x) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k.v[x], q.v[x], acc, 0, 0, 0);
        return acc;
    }
    // O tile (16 queries x 16 dims) += P (16 q x 16 keys) . V (16 keys x 16 dims)
    // p[r]: weight of key 4*grp + r for query r16. vk: V rows of keys 4*grp + r, this lane's dim.
    __device__ static v4f pv(const float p[4], const float* vbase, size_t vstride[4], int dim, v4f acc) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(p[r], vbase[vstride[r] + dim], acc, 0, 0, 0);
        return acc;
    }
};

// bf16: lane l covers dims [DPL*grp, DPL*grp + DPL), DPL = D/4 (4 or 8), in MFMA
// steps of 4 bf16.
template <int D>
struct DenseOps<uint16_t, D> {
    static constexpr int DPL = D / 4;
    struct Row { v4s v[DPL / 4]; };
    __device__ static Row load(const uint16_t* row, int grp) {
        Row r;
        const uint16_t* src = row + grp * DPL;
#pragma unroll
        for (int x = 0; x < DPL / 4; ++x) {
            const uint2 u = *reinterpret_cast<const uint2*>(src + 4 * x);
            r.v[x][0] = (short)(u.x & 0xFFFF); r.v[x][1] = (short)(u.x >> 16);
            r.v[x][2] = (short)(u.y & 0xFFFF); r.v[x][3] = (short)(u.y >> 16);
        }
        return r;
    }
    __device__ static v4f scores(const Row& k, const Row& q) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int x = 0; x < DPL / 4; ++x)
            acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(k.v[x], q.v[x], acc, 0, 0, 0);
        return acc;
    }
    __device__ static v4f pv(const float p[4], const uint16_t* vbase, size_t vstride[4], int dim, v4f acc) {
        v4s hi, lo, vv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t h = f32_to_bf16_bits(p[r]);
            const float rem = p[r] - __uint_as_float(h << 16);
            hi[r] = (short)h;
            lo[r] = (short)f32_to_bf16_bits(rem);
            vv[r] = (short)vbase[vstride[r] + dim];
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, vv, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, vv, acc, 0, 0, 0);
        return acc;
    }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void dense_layer_kernel(const DenseArgs p) {
    using Ops = DenseOps<T, D>;
    const Geom g = p.g;
    const int N = g.N;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    const int qblocks = (N + 63) / 64;
    const int wh = blockIdx.x / qblocks;
    const int q0 = (blockIdx.x - wh * qblocks) * 64 + wave * 16;
    if (q0 >= N) return;
    const int nwin = g.nwy * g.nwx;
    const int win_id = wh % nwin;
    const int bh = wh / nwin;
    const int wy = win_id / g.nwx;
    const int wx = win_id - wy * g.nwx;
    const size_t plane = (size_t)bh * g.H * g.W * D;
    const T* Qh = static_cast<const T*>(p.Q) + plane;
    const T* Kh = static_cast<const T*>(p.K) + plane;
    const T* Vh = static_cast<const T*>(p.V) + plane;
    float* Oh = p.O_out + plane;
    const float sc = p.scale2;

    const typename Ops::Row qop = Ops::load(Qh + (size_t)slot_pixel(g, wy, wx, q0 + r16) * D, grp);
    const int ntiles = N / 16;

    // pass 1: per-lane running max / sum over the keys 4*grp + r of every tile
    float m = -INFINITY, l = 0.0f;
    for (int kt = 0; kt < ntiles; ++kt) {
        const typename Ops::Row kop = Ops::load(Kh + (size_t)slot_pixel(g, wy, wx, kt * 16 + r16) * D, grp);
        const v4f acc = Ops::scores(kop, qop);
        const float s0 = acc[0] * sc, s1 = acc[1] * sc, s2 = acc[2] * sc, s3 = acc[3] * sc;
        const float mn = fmaxf(m, fmaxf(fmaxf(s0, s1), fmaxf(s2, s3)));
        l = l * fast_exp2(m - mn) + fast_exp2(s0 - mn) + fast_exp2(s1 - mn) + fast_exp2(s2 - mn) +
            fast_exp2(s3 - mn);
        m = mn;
    }
    // combine the 4 lane groups holding the same query
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
        const float m2 = __shfl_xor(m, o);
        const float l2 = __shfl_xor(l, o);
        const float mn = fmaxf(m, m2);
        l = l * fast_exp2(m - mn) + l2 * fast_exp2(m2 - mn);
        m = mn;
    }
    const float inv_l = 1.0f / l;

    // pass 2: probabilities, A^1 rows, O += P V
    constexpr int CT = D / 16;
    v4f oacc[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) oacc[c] = v4f{0.f, 0.f, 0.f, 0.f};
    float* Arow = p.A_out ? p.A_out + ((size_t)wh * N + q0 + r16) * N : nullptr;
    for (int kt = 0; kt < ntiles; ++kt) {
        const typename Ops::Row kop = Ops::load(Kh + (size_t)slot_pixel(g, wy, wx, kt * 16 + r16) * D, grp);
        const v4f acc = Ops::scores(kop, qop);
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(acc[r] * sc - m) * inv_l;
        if (Arow)
            *reinterpret_cast<float4*>(Arow + kt * 16 + 4 * grp) = make_float4(pr[0], pr[1], pr[2], pr[3]);
        size_t vrow[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) vrow[r] = (size_t)slot_pixel(g, wy, wx, kt * 16 + 4 * grp + r) * D;
#pragma unroll
        for (int c = 0; c < CT; ++c) oacc[c] = Ops::pv(pr, Vh, vrow, c * 16 + r16, oacc[c]);
    }
    // lane holds O[query q0 + 4*grp + r][dim 16c + r16]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float* orow = Oh + (size_t)slot_pixel(g, wy, wx, q0 + 4 * grp + r) * D;
#pragma unroll
        for (int c = 0; c < CT; ++c) orow[c * 16 + r16] = oacc[c][r];
    }
}

__global__ void iota_rows_kernel(int32_t* I, int64_t total, int N) {
    for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < total;
         x += (int64_t)gridDim.x * blockDim.x)
        I[x] = (int32_t)(x % N);
}

}  // namespace

hipError_t launch_dense(const DenseArgs& a, int dtype, int D, int grid, hipStream_t stream) {
    if (dtype == 0) {
        if (D == 16) hipLaunchKernelGGL((dense_layer_kernel<float, 16>), dim3(grid), dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((dense_layer_kernel<float, 32>), dim3(grid), dim3(256), 0, stream, a);
    } else {
        if (D == 16) hipLaunchKernelGGL((dense_layer_kernel<uint16_t, 16>), dim3(grid), dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((dense_layer_kernel<uint16_t, 32>), dim3(grid), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_iota_rows(int32_t* I, int64_t rows, int N, hipStream_t stream) {
    const int64_t total = rows * N;
    int grid = (int)((total + 255) / 256);
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(iota_rows_kernel, dim3(grid), dim3(256), 0, stream, I, total, N);
    return hipGetLastError();
}

}  // namespace pfa
