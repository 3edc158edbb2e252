// Sparse PFA layer on gfx950: one wavefront per query row.
//
// Per window-head and query slot i (paper notes "Progressive Focused Transformer
// for Single Image Super-Resolution", sections "Progressive attention across
// layers" and "Sparse matrix multiplication"):
//   s_ij  = q_i . k_j / sqrt(d)           only for j in I^{l-1}(i)
//   u_ij  = A^{l-1}_ij * exp(s_ij - m_i)  (softmax and the first Norm are row
//                                          constants and do not change the order)
//   keep the K_l largest u (ties to the lower j), A^l = u / sum_kept u,
//   O_i   = sum_kept A^l_ij v_j.
//
// Dataflow: the window's K rows (and V rows when they fit) are staged once in
// LDS in slot order, so the cyclic shift costs nothing after staging. Each wave
// then walks its query rows: lane L owns candidates c = L + 64t (coalesced loads
// of the I^{l-1}/A^{l-1} rows), gathers k_j from LDS reading the 16-byte chunks
// of the row in a lane-rotated order (8 consecutive lanes always touch 8
// different chunks, so a 128-byte fp32 row never bank-conflicts), selects the
// top K_l exactly by bisection on the fp32 bit patterns of u (counts via
// ballot + popcount), compacts the kept entries in I^{l-1} order (ballot +
// mbcnt) and aggregates V with CH lanes per row chunk.
#include "pfa_kernels.h"

namespace pfa {
namespace {

template <typename T>
struct Chunk;

template <>
struct Chunk<float> {
    static constexpr int kElems = 4;
    __device__ static void to_f32(const uint4 c, float* o) {
        o[0] = __uint_as_float(c.x);
        o[1] = __uint_as_float(c.y);
        o[2] = __uint_as_float(c.z);
        o[3] = __uint_as_float(c.w);
    }
};

template <>
struct Chunk<uint16_t> {  // bf16 bit patterns
    static constexpr int kElems = 8;
    __device__ static void to_f32(const uint4 c, float* o) {
        o[0] = bf16_lo(c.x); o[1] = bf16_hi(c.x);
        o[2] = bf16_lo(c.y); o[3] = bf16_hi(c.y);
        o[4] = bf16_lo(c.z); o[5] = bf16_hi(c.z);
        o[6] = bf16_lo(c.w); o[7] = bf16_hi(c.w);
    }
};

template <typename T, int D, int KPT, int MODE>
__global__ __launch_bounds__(kSparseWaves * kWave) void sparse_layer_kernel(const SparseArgs p) {
    constexpr int EPC = Chunk<T>::kElems;   // elements per 16-byte chunk
    constexpr int CH = D / EPC;             // chunks per K/V row
    constexpr int ROWB = D * (int)sizeof(T);
    constexpr int G = kWave / CH;           // lane groups in the aggregation
    constexpr bool K_LDS = MODE != kKVglobal;
    constexpr bool V_LDS = MODE == kKVinLDS;
    extern __shared__ __align__(16) unsigned char smem[];

    const Geom g = p.g;
    const int N = g.N;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int wh = blockIdx.x / p.blocks_per_wh;
    const int part = blockIdx.x - wh * p.blocks_per_wh;
    const int nwin = g.nwy * g.nwx;
    const int win_id = wh % nwin;
    const int bh = wh / nwin;
    const int b = bh / g.heads;
    const int wy = win_id / g.nwx;
    const int wx = win_id - wy * g.nwx;
    const size_t plane = (size_t)bh * g.H * g.W * D;
    const T* Qh = static_cast<const T*>(p.Q) + plane;
    const T* Kh = static_cast<const T*>(p.K) + plane;
    const T* Vh = static_cast<const T*>(p.V) + plane;
    float* Oh = p.O_out + plane;

    unsigned char* Ks = smem;
    unsigned char* Vs = smem + (K_LDS ? N * ROWB : 0);
    uint2* scratch = reinterpret_cast<uint2*>(smem + (K_LDS ? N * ROWB : 0) + (V_LDS ? N * ROWB : 0)) +
                     wave * kScratchEntries;

    if (K_LDS) {
        for (int u = threadIdx.x; u < N * CH; u += blockDim.x) {
            const int t = u / CH;
            const int c = u - t * CH;
            const size_t src = (size_t)slot_pixel(g, wy, wx, t) * D + c * EPC;
            *reinterpret_cast<uint4*>(Ks + t * ROWB + c * 16) = *reinterpret_cast<const uint4*>(Kh + src);
            if (V_LDS)
                *reinterpret_cast<uint4*>(Vs + t * ROWB + c * 16) = *reinterpret_cast<const uint4*>(Vh + src);
        }
        __syncthreads();
    }

    // lane-rotated chunk order for gathers of whole rows
    int coff[CH];
#pragma unroll
    for (int m = 0; m < CH; ++m) coff[m] = ((m + lane) % CH) * 16;
    const int vchunk = lane % CH;           // aggregation: chunk of the V row owned by this lane
    const int vgroup = lane / CH;

    const int row0 = part * p.rows_per_block;
    const int row1 = min(N, row0 + p.rows_per_block);
    const int K_prev = p.K_prev;
    const int K_l = p.K_l;

    for (int i = row0 + wave; i < row1; i += kSparseWaves) {
        const int qpix = slot_pixel(g, wy, wx, i);
        const size_t row = (size_t)wh * N + i;                       // I/A/out row
        const size_t rowI = p.i_shared ? (size_t)(b * nwin + win_id) * N + i : row;

        // candidates of this lane, previous weights
        int jj[KPT];
        float av[KPT];
#pragma unroll
        for (int t = 0; t < KPT; ++t) {
            const int c = lane + kWave * t;
            const bool valid = c < K_prev;
            const int j = valid ? (p.I_prev ? p.I_prev[rowI * K_prev + c] : c) : 0;
            jj[t] = min(max(j, 0), N - 1);   // memory safety only: indices must lie in [0, N)
            av[t] = (valid && p.A_prev) ? p.A_prev[row * K_prev + c] : 1.0f;
        }

        // q_i in the lane-rotated chunk order
        float qf[D];
        const unsigned char* qrow = reinterpret_cast<const unsigned char*>(Qh + (size_t)qpix * D);
#pragma unroll
        for (int m = 0; m < CH; ++m)
            Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(qrow + coff[m]), &qf[m * EPC]);

        // SMM: scores over the candidate list only (base-2 units)
        float sv[KPT];
        float smax = -INFINITY;
#pragma unroll
        for (int t = 0; t < KPT; ++t) {
            const unsigned char* krow =
                K_LDS ? Ks + jj[t] * ROWB
                      : reinterpret_cast<const unsigned char*>(Kh + (size_t)jj[t] * D);
            float acc = 0.0f;
#pragma unroll
            for (int m = 0; m < CH; ++m) {
                float kf[EPC];
                Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(krow + coff[m]), kf);
#pragma unroll
                for (int e = 0; e < EPC; ++e) acc = fmaf(qf[m * EPC + e], kf[e], acc);
            }
            const bool valid = lane + kWave * t < K_prev;
            sv[t] = valid ? acc * p.scale2 : -INFINITY;
            smax = fmaxf(smax, sv[t]);
        }
        smax = wave_max(smax);

        // u = A^{l-1} * exp(s - m); keys are the fp32 bit patterns (u >= 0), -1 = no candidate
        float uv[KPT];
        int key[KPT];
        int kmin = 0x7fffffff, kmax = -1;
#pragma unroll
        for (int t = 0; t < KPT; ++t) {
            const bool valid = lane + kWave * t < K_prev;
            uv[t] = valid ? av[t] * fast_exp2(sv[t] - smax) : 0.0f;
            key[t] = valid ? __float_as_int(uv[t]) : -1;
            if (valid) {
                kmin = min(kmin, key[t]);
                kmax = max(kmax, key[t]);
            }
        }
        kmin = __builtin_amdgcn_readfirstlane(wave_min_i(kmin));
        kmax = __builtin_amdgcn_readfirstlane(wave_max_i(kmax));

        // exact K_l-th largest key: count(key >= lo) >= K_l > count(key >= hi)
        int lo = kmin, hi = kmax + 1, c_hi = 0;
        while (hi - lo > 1) {
            const int mid = lo + ((hi - lo) >> 1);
            int cnt = 0;
#pragma unroll
            for (int t = 0; t < KPT; ++t) cnt += popc(ballot(key[t] >= mid));
            if (cnt >= K_l) {
                lo = mid;
            } else {
                hi = mid;
                c_hi = cnt;
            }
        }
        const int tau = lo;
        const int need = K_l - c_hi;   // entries equal to tau that are kept
        int n_eq = 0;
#pragma unroll
        for (int t = 0; t < KPT; ++t) n_eq += popc(ballot(key[t] == tau));
        int jcut = 0x7fffffff;
        if (n_eq > need) {   // exact ties at the boundary: keep the lowest slot indices
            int jl = -1, jh = N - 1;
            while (jh - jl > 1) {
                const int mid = (jl + jh) >> 1;
                int cnt = 0;
#pragma unroll
                for (int t = 0; t < KPT; ++t) cnt += popc(ballot(key[t] == tau && jj[t] <= mid));
                if (cnt >= need) jh = mid; else jl = mid;
            }
            jcut = jh;
        }

        bool kept[KPT];
        float ksum = 0.0f;
#pragma unroll
        for (int t = 0; t < KPT; ++t) {
            kept[t] = key[t] > tau || (key[t] == tau && jj[t] <= jcut);
            ksum += kept[t] ? uv[t] : 0.0f;
        }
        const float inv = 1.0f / wave_sum(ksum);

        // kept entries in I^{l-1} order
        int pos[KPT];
        int base = 0;
        int32_t* Io = p.I_out + row * K_l;
        float* Ao = p.A_out + row * K_l;
#pragma unroll
        for (int t = 0; t < KPT; ++t) {
            const uint64_t m = ballot(kept[t]);
            pos[t] = kept[t] ? base + lanes_below(m) : -1;
            uv[t] *= inv;
            if (kept[t] && pos[t] < K_l) {   // < K_l always holds for distinct indices
                Io[pos[t]] = jj[t];
                Ao[pos[t]] = uv[t];
            }
            base += popc(m);
        }

        // O_i = sum_kept A v_j: lane owns chunk vchunk of the rows of entries vgroup, vgroup+G, ...
        float oacc[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) oacc[e] = 0.0f;
        for (int P0 = 0; P0 < K_l; P0 += kScratchEntries) {
#pragma unroll
            for (int t = 0; t < KPT; ++t)
                if (pos[t] >= P0 && pos[t] < P0 + kScratchEntries && pos[t] < K_l)
                    scratch[pos[t] - P0] = make_uint2((uint32_t)jj[t], __float_as_uint(uv[t]));
            __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            const int cnt = min(kScratchEntries, K_l - P0);
            for (int e = vgroup; e < cnt; e += G) {
                const uint2 ent = scratch[e];
                const float w = __uint_as_float(ent.y);
                const unsigned char* vrow;
                if (V_LDS) {
                    vrow = Vs + ent.x * ROWB;
                } else if (K_LDS) {
                    vrow = reinterpret_cast<const unsigned char*>(
                        Vh + (size_t)slot_pixel(g, wy, wx, (int)ent.x) * D);
                } else {
                    vrow = reinterpret_cast<const unsigned char*>(Vh + (size_t)ent.x * D);
                }
                float vf[EPC];
                Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(vrow + vchunk * 16), vf);
#pragma unroll
                for (int x = 0; x < EPC; ++x) oacc[x] = fmaf(w, vf[x], oacc[x]);
            }
            __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
#pragma unroll
        for (int o = CH; o < kWave; o <<= 1)
#pragma unroll
            for (int x = 0; x < EPC; ++x) oacc[x] += __shfl_xor(oacc[x], o);
        if (vgroup == 0) {
            float* orow = Oh + (size_t)qpix * D + vchunk * EPC;
#pragma unroll
            for (int x = 0; x < EPC; x += 4)
                *reinterpret_cast<float4*>(orow + x) = make_float4(oacc[x], oacc[x + 1], oacc[x + 2], oacc[x + 3]);
        }
    }
}

template <typename T, int D, int KPT, int MODE>
hipError_t launch_one(const SparseArgs& a, int lds, int grid, hipStream_t s) {
    auto fn = sparse_layer_kernel<T, D, KPT, MODE>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(kSparseWaves * kWave), lds, s, a);
    return hipGetLastError();
}

template <typename T, int D, int KPT>
hipError_t launch_mode(const SparseArgs& a, SparseMode mode, int lds, int grid, hipStream_t s) {
    switch (mode) {
        case kKVinLDS: return launch_one<T, D, KPT, kKVinLDS>(a, lds, grid, s);
        case kKinLDS: return launch_one<T, D, KPT, kKinLDS>(a, lds, grid, s);
        default: return launch_one<T, D, KPT, kKVglobal>(a, lds, grid, s);
    }
}

template <typename T, int D>
hipError_t launch_kpt(const SparseArgs& a, int kpt, SparseMode mode, int lds, int grid, hipStream_t s) {
    switch (kpt) {
        case 1: return launch_mode<T, D, 1>(a, mode, lds, grid, s);
        case 2: return launch_mode<T, D, 2>(a, mode, lds, grid, s);
        case 4: return launch_mode<T, D, 4>(a, mode, lds, grid, s);
        case 8: return launch_mode<T, D, 8>(a, mode, lds, grid, s);
        default: return launch_mode<T, D, 16>(a, mode, lds, grid, s);
    }
}

}  // namespace

hipError_t launch_sparse(const SparseArgs& a, int dtype, int D, int kpt, SparseMode mode, int lds_bytes,
                         int grid, hipStream_t stream) {
    if (dtype == 0)
        return D == 16 ? launch_kpt<float, 16>(a, kpt, mode, lds_bytes, grid, stream)
                       : launch_kpt<float, 32>(a, kpt, mode, lds_bytes, grid, stream);
    return D == 16 ? launch_kpt<uint16_t, 16>(a, kpt, mode, lds_bytes, grid, stream)
                   : launch_kpt<uint16_t, 32>(a, kpt, mode, lds_bytes, grid, stream);
}

}  // namespace pfa
