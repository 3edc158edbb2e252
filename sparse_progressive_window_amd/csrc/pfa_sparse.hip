// Sparse PFA layer on gfx950.
//
// Per window-head and query slot i (paper notes "Progressive Focused Transformer
// for Single Image Super-Resolution", sections "Progressive attention across
// layers" and "Sparse matrix multiplication"):
//   s_ij  = q_i . k_j / sqrt(d)           only for j in I^{l-1}(i)
//   u_ij  = A^{l-1}_ij * exp(s_ij - m_i)  (softmax and the first Norm are row
//                                          constants: they do not change the order)
//   keep the K_l largest u (ties to the lower j), A^l = u / sum_kept u,
//   O_i   = sum_kept A^l_ij v_j.
//
// Dataflow. The window's K rows (and V rows when they fit) are staged once per
// workgroup in LDS in slot order, so the cyclic shift costs nothing after
// staging. A query row is handled by a group of GL lanes (GL = 16, 32 or 64,
// the smallest power of two >= K_prev/4, so a wavefront handles 64/GL rows at
// once); lane l of the group owns candidates c = l + GL*t (coalesced loads of
// the I^{l-1} / A^{l-1} rows). k_j is gathered from LDS reading the 16-byte
// chunks of the row in a lane-rotated order, so 8 consecutive lanes always touch
// 8 different chunks and a 128-byte row never bank-conflicts.
//
// Top-K. Keys are the fp32 bit patterns of u (u >= 0, so integer order = float
// order). A search on the key interval [lo, hi) with count(key >= lo) >= K_l >
// count(key >= hi) narrows the interval by interpolation in bit space (that is,
// in log u), with a bisection step every third iteration, until at most kBand
// keys remain in it; those are then extracted largest first. Counts use wave
// ballots; every reduction inside a group uses DPP (quad permutes, row
// rotations), ds_swizzle for the 16-lane half swap and readlane across halves.
// Ties at the threshold keep the lowest slot indices (bisection on j).
//
// Kept entries are compacted in I^{l-1} order (ballot + lane-prefix counts) and
// staged in LDS as (j, weight); the aggregation then gives each V row chunk to
// a lane (CH lanes read one whole row, conflict-free) and sums the lanes of a
// group with row rotations.
#include "pfa_kernels.h"

namespace pfa {
namespace {

constexpr int kBand = 8;

// DPP controls (GFX9 encoding)
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowRor2 = 0x122;
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(dpp<CTRL>(__float_as_int(v)));
}
__device__ __forceinline__ int swap16(int v) { return __builtin_amdgcn_ds_swizzle(v, 0x401F); }
__device__ __forceinline__ float swap16f(float v) { return __int_as_float(swap16(__float_as_int(v))); }

struct MaxF { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct SumF { __device__ float operator()(float a, float b) const { return a + b; } };
struct MaxI { __device__ int operator()(int a, int b) const { return max(a, b); } };
struct MinI { __device__ int operator()(int a, int b) const { return min(a, b); } };

// Reductions and counts over a group of GL consecutive lanes; every lane of the
// group receives the result.
template <int GL>
struct Grp {
    template <class Op>
    __device__ static float all(float v, Op op) {
        v = op(v, dppf<kQuadXor1>(v));
        v = op(v, dppf<kQuadXor2>(v));
        v = op(v, dppf<kRowRor4>(v));
        v = op(v, dppf<kRowRor8>(v));
        if (GL >= 32) v = op(v, swap16f(v));
        if (GL == 64)
            v = op(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
                   __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)));
        return v;
    }
    template <class Op>
    __device__ static int all_i(int v, Op op) {
        v = op(v, dpp<kQuadXor1>(v));
        v = op(v, dpp<kQuadXor2>(v));
        v = op(v, dpp<kRowRor4>(v));
        v = op(v, dpp<kRowRor8>(v));
        if (GL >= 32) v = op(v, swap16(v));
        if (GL == 64) v = op(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 32));
        return v;
    }
    // bits of the wave mask m that belong to this lane's group
    __device__ static uint32_t bits(uint64_t m, int lane) {
        if (GL == 64) return 0;  // unused
        const uint32_t half = (lane & 32) ? (uint32_t)(m >> 32) : (uint32_t)m;
        if (GL == 32) return half;
        return (half >> (lane & 16)) & 0xFFFFu;
    }
    __device__ static int count_mask(uint64_t m, int lane) {
        if (GL == 64) return popc(m);
        return __builtin_popcount(bits(m, lane));
    }
    __device__ static int count(bool p, int lane) { return count_mask(ballot(p), lane); }
    // set bits of m in this group at lanes below this lane
    __device__ static int below(uint64_t m, int lane) {
        if (GL == 64) return lanes_below(m);
        const uint32_t b = bits(m, lane);
        return __builtin_popcount(b & ((1u << (lane & (GL - 1))) - 1u));
    }
};

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

// sum the lanes of a group that own the same chunk (lane bits [log2 CH, log2 GL))
template <int CH, int GL>
__device__ __forceinline__ float reduce_chunk_lanes(float v) {
    if (CH <= 2) v += dppf<kRowRor2>(v);
    if (CH <= 4 && GL >= 8) v += dppf<kRowRor4>(v);
    if (CH <= 8 && GL >= 16) v += dppf<kRowRor8>(v);
    if (GL >= 32) v += swap16f(v);
    if (GL == 64) v += __shfl_xor(v, 32);
    return v;
}

template <typename T, int D, int GL, int KPT, int MODE, int NW>
__global__ __launch_bounds__(NW * kWave) void sparse_layer_kernel(const SparseArgs p) {
    constexpr int EPC = Chunk<T>::kElems;   // elements per 16-byte chunk
    constexpr int CH = D / EPC;             // chunks per K/V row
    constexpr int ROWB = D * (int)sizeof(T);
    constexpr int RPW = kWave / GL;         // rows per wavefront iteration
    constexpr int GS = GL / CH;             // lanes sharing a V chunk in the aggregation
    constexpr bool K_LDS = MODE != kKVglobal;
    constexpr bool V_LDS = MODE == kKVinLDS;
    constexpr int SCW = kScratchBytes / (NW * 8);   // scratch entries per wave
    constexpr int SCG = SCW / RPW;                  // scratch entries per row group
    using G = Grp<GL>;
    extern __shared__ __align__(16) unsigned char smem[];

    const Geom g = p.g;
    const int N = g.N;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int grp = lane / GL;
    const int gl = lane & (GL - 1);

    // workgroup -> (window-head, part); parts of one window-head share an XCD
    int wh, part;
    if (p.xcd_map) {
        const int xcd = blockIdx.x & 7;
        const int slot = blockIdx.x >> 3;
        part = slot % p.blocks_per_wh;
        wh = (slot / p.blocks_per_wh) * 8 + xcd;
    } else {
        wh = blockIdx.x / p.blocks_per_wh;
        part = blockIdx.x - wh * p.blocks_per_wh;
    }
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
    uint2* scr = reinterpret_cast<uint2*>(smem + (K_LDS ? N * ROWB : 0) + (V_LDS ? N * ROWB : 0)) +
                 wave * SCW + grp * SCG;

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

    int coff[CH];   // lane-rotated chunk order for whole-row gathers
#pragma unroll
    for (int m = 0; m < CH; ++m) coff[m] = ((m + lane) % CH) * 16;
    const int vchunk = gl % CH;
    const int vsub = gl / CH;

    const int row0 = part * p.rows_per_block;
    const int row1 = min(N, row0 + p.rows_per_block);
    const int K_prev = p.K_prev;
    const int K_l = p.K_l;

    for (int base = row0 + wave * RPW; base < row1; base += NW * RPW) {
        const int i_raw = base + grp;
        const bool active = i_raw < row1;
        const int i = active ? i_raw : row0;
        const int qpix = slot_pixel(g, wy, wx, i);
        const size_t row = (size_t)wh * N + i;
        const size_t rowI = p.i_shared ? (size_t)(b * nwin + win_id) * N + i : row;

        int jj[KPT];
        float av[KPT];
        bool valid[KPT];
#pragma unroll
        for (int t = 0; t < KPT; ++t) {
            const int c = gl + GL * t;
            valid[t] = active && c < K_prev;
            const int j = valid[t] ? (p.I_prev ? p.I_prev[rowI * K_prev + c] : c) : 0;
            jj[t] = min(max(j, 0), N - 1);   // memory safety only: indices must lie in [0, N)
            av[t] = (valid[t] && p.A_prev) ? p.A_prev[row * K_prev + c] : 1.0f;
        }

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
                K_LDS ? Ks + jj[t] * ROWB : reinterpret_cast<const unsigned char*>(Kh + (size_t)jj[t] * D);
            float acc = 0.0f;
#pragma unroll
            for (int m = 0; m < CH; ++m) {
                float kf[EPC];
                Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(krow + coff[m]), kf);
#pragma unroll
                for (int e = 0; e < EPC; ++e) acc = fmaf(qf[m * EPC + e], kf[e], acc);
            }
            sv[t] = valid[t] ? acc * p.scale2 : -INFINITY;
            smax = fmaxf(smax, sv[t]);
        }
        smax = G::all(smax, MaxF());

        // u = A^{l-1} exp(s - m); key = bits of u (>= 0), -1 for no candidate
        float uv[KPT];
        int key[KPT];
        int kmin = 0x7fffffff, kmax = -1;
#pragma unroll
        for (int t = 0; t < KPT; ++t) {
            uv[t] = valid[t] ? av[t] * fast_exp2(sv[t] - smax) : 0.0f;
            key[t] = valid[t] ? __float_as_int(uv[t]) : -1;
            if (valid[t]) {
                kmin = min(kmin, key[t]);
                kmax = max(kmax, key[t]);
            }
        }
        kmin = G::all_i(kmin, MinI());
        kmax = G::all_i(kmax, MaxI());

        // phase 1: narrow [lo, hi) until it holds at most kBand keys
        int lo = kmin, hi = kmax + 1, c_lo = K_prev, c_hi = 0;
        bool done = !active || hi - lo <= 1 || c_lo - c_hi <= kBand;
        for (int it = 0; ballot(!done) != 0; ++it) {
            const int span = hi - lo;
            int mid;
            if (it % 3 == 2) {
                mid = lo + (span >> 1);
            } else {
                const float f = ((float)(c_lo - K_l) + 0.5f) / (float)max(c_lo - c_hi, 1);
                mid = lo + (int)(f * (float)span);
            }
            mid = min(max(mid, lo + 1), hi - 1);
            int cnt = 0;
#pragma unroll
            for (int t = 0; t < KPT; ++t) cnt += G::count(key[t] >= mid, lane);
            if (!done) {
                if (cnt >= K_l) { lo = mid; c_lo = cnt; } else { hi = mid; c_hi = cnt; }
                done = hi - lo <= 1 || c_lo - c_hi <= kBand;
            }
        }

        // phase 2: take the band's keys largest first until K_l are kept
        int need = K_l - c_hi;
        int tau = lo, need_tau = need, n_tau = 0;
        bool done2 = !active;
        while (ballot(!done2) != 0) {
            int m = -1;
#pragma unroll
            for (int t = 0; t < KPT; ++t)
                if (key[t] >= lo && key[t] < hi) m = max(m, key[t]);
            m = G::all_i(m, MaxI());
            int ceq = 0;
#pragma unroll
            for (int t = 0; t < KPT; ++t) ceq += G::count(key[t] == m, lane);
            if (!done2) {
                if (ceq >= need) {
                    tau = m; need_tau = need; n_tau = ceq; done2 = true;
                } else {
                    need -= ceq; hi = m;
                }
            }
        }

        // exact ties at the threshold: keep the lowest slot indices
        int jcut = 0x7fffffff;
        const bool tie = active && n_tau > need_tau;
        if (ballot(tie) != 0) {
            int jl = -1, jh = N - 1;
            while (ballot(tie && jh - jl > 1) != 0) {
                const int mid = (jl + jh) >> 1;
                int cnt = 0;
#pragma unroll
                for (int t = 0; t < KPT; ++t) cnt += G::count(key[t] == tau && jj[t] <= mid, lane);
                if (tie && jh - jl > 1) {
                    if (cnt >= need_tau) jh = mid; else jl = mid;
                }
            }
            if (tie) jcut = jh;
        }

        bool kept[KPT];
        float ksum = 0.0f;
#pragma unroll
        for (int t = 0; t < KPT; ++t) {
            kept[t] = key[t] > tau || (key[t] == tau && jj[t] <= jcut);
            ksum += kept[t] ? uv[t] : 0.0f;
        }
        const float inv = 1.0f / G::all(ksum, SumF());

        // kept entries in I^{l-1} order
        int pos[KPT];
        int obase = 0;
        int32_t* Io = p.I_out + row * K_l;
        float* Ao = p.A_out + row * K_l;
#pragma unroll
        for (int t = 0; t < KPT; ++t) {
            const uint64_t m = ballot(kept[t]);
            pos[t] = kept[t] ? obase + G::below(m, lane) : -1;
            if (pos[t] >= K_l) pos[t] = -1;   // only on precondition violations
            uv[t] *= inv;
            if (pos[t] >= 0) {
                Io[pos[t]] = jj[t];
                Ao[pos[t]] = uv[t];
            }
            obase += G::count_mask(m, lane);
        }

        // O_i = sum_kept A v_j
        float oacc[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) oacc[e] = 0.0f;
        for (int P0 = 0; P0 < K_l; P0 += SCG) {
#pragma unroll
            for (int t = 0; t < KPT; ++t)
                if (pos[t] >= P0 && pos[t] < P0 + SCG)
                    scr[pos[t] - P0] = make_uint2((uint32_t)jj[t], __float_as_uint(uv[t]));
            __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            const int cnt = active ? min(SCG, K_l - P0) : 0;
            for (int e = vsub; e < cnt; e += GS) {
                const uint2 ent = scr[e];
                const float w = __uint_as_float(ent.y);
                const unsigned char* vrow;
                if (V_LDS) {
                    vrow = Vs + ent.x * ROWB;
                } else if (K_LDS) {
                    vrow = reinterpret_cast<const unsigned char*>(Vh + (size_t)slot_pixel(g, wy, wx, (int)ent.x) * D);
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
        for (int x = 0; x < EPC; ++x) oacc[x] = reduce_chunk_lanes<CH, GL>(oacc[x]);
        if (active && vsub == 0) {
            float* orow = Oh + (size_t)qpix * D + vchunk * EPC;
#pragma unroll
            for (int x = 0; x < EPC; x += 4)
                *reinterpret_cast<float4*>(orow + x) = make_float4(oacc[x], oacc[x + 1], oacc[x + 2], oacc[x + 3]);
        }
    }
}

template <typename T, int D, int GL, int KPT, int MODE>
hipError_t launch_one(const SparseArgs& a, int lds, int grid, hipStream_t s) {
    constexpr int NW = KPT <= 4 ? 16 : 8;
    auto fn = sparse_layer_kernel<T, D, GL, KPT, MODE, NW>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(NW * kWave), lds, s, a);
    return hipGetLastError();
}

template <typename T, int D, int GL, int KPT>
hipError_t launch_mode(const SparseArgs& a, SparseMode mode, int lds, int grid, hipStream_t s) {
    switch (mode) {
        case kKVinLDS: return launch_one<T, D, GL, KPT, kKVinLDS>(a, lds, grid, s);
        case kKinLDS: return launch_one<T, D, GL, KPT, kKinLDS>(a, lds, grid, s);
        default: return launch_one<T, D, GL, KPT, kKVglobal>(a, lds, grid, s);
    }
}

template <typename T, int D>
hipError_t launch_shape(const SparseArgs& a, SparseMode mode, int lds, int grid, hipStream_t s) {
    const int kp = a.K_prev;
    if (kp <= 16) return launch_mode<T, D, 16, 1>(a, mode, lds, grid, s);
    if (kp <= 32) return launch_mode<T, D, 16, 2>(a, mode, lds, grid, s);
    if (kp <= 64) return launch_mode<T, D, 16, 4>(a, mode, lds, grid, s);
    if (kp <= 128) return launch_mode<T, D, 32, 4>(a, mode, lds, grid, s);
    if (kp <= 256) return launch_mode<T, D, 64, 4>(a, mode, lds, grid, s);
    if (kp <= 512) return launch_mode<T, D, 64, 8>(a, mode, lds, grid, s);
    return launch_mode<T, D, 64, 16>(a, mode, lds, grid, s);
}

}  // namespace

hipError_t launch_sparse(const SparseArgs& a, int dtype, int D, SparseMode mode, int lds_bytes, int grid,
                         hipStream_t stream) {
    if (dtype == 0)
        return D == 16 ? launch_shape<float, 16>(a, mode, lds_bytes, grid, stream)
                       : launch_shape<float, 32>(a, mode, lds_bytes, grid, stream);
    return D == 16 ? launch_shape<uint16_t, 16>(a, mode, lds_bytes, grid, stream)
                   : launch_shape<uint16_t, 32>(a, mode, lds_bytes, grid, stream);
}

}  // namespace pfa
