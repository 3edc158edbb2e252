// Dense first PFA layer on gfx950 matrix cores.
//
// The first layer keeps every token of the window and computes the complete
// softmax map (paper notes "Progressive Focused Transformer for Single Image
// Super-Resolution", section "Progressive focused resource allocation
// strategy"): A^1 = softmax(Q K^T / sqrt(d)) per window-head, O = A^1 V.
//
// A workgroup of 8 waves owns 128 query rows of one window-head (16 per wave);
// K and V stream through LDS in tiles of 64 keys, double-buffered, shared by
// all 8 waves (rows padded by 16 bytes so the MFMA operand reads of 16
// consecutive rows hit distinct banks). The global loads run two tiles ahead
// in two register sets, so each has two tiles of work to land. The workgroups
// of one window-head are consecutive on one XCD, so its K/V stay in that XCD's
// L2.
//
// Scores are produced transposed, S^T = K Q^T, with 16x16 MFMA tiles (16 keys x
// 16 queries): the accumulator gives each lane 4 consecutive keys of one query,
// which is exactly the A-operand layout of the following P.V MFMA, so the
// probabilities never leave registers. The contraction index of the score
// MFMAs is permuted so every lane reads a contiguous run of d/4 elements.
//   fp32 inputs, d = 32, 64-key tiles: the scores use v_mfma_f32_16x16x32_bf16
//   on a three-way bf16 split of q and k (x = x_hi + x_mid + x_lo, each part the
//   round-to-nearest bf16 of what is left, so |x - sum| <= 2^-24 |x|); the six
//   products down to order 2^-16 are accumulated smallest first and the dropped
//   ones are below 2^-26 of |q||k|: scores as accurate as fp32 products, at 6
//   bf16 MFMAs instead of 8 fp32 ones per 16x16 tile. K is split once, when its
//   tile is staged in LDS (three bf16 planes). P.V stays on fp32 MFMA.
//   fp32 inputs otherwise: v_mfma_f32_16x16x4_f32 (exact products, fp32 accumulation).
//   bf16 inputs: v_mfma_f32_16x16x16_bf16; P is split into bf16 hi + lo parts
//   (two MFMAs, the split done once per 16-key tile with the hardware
//   conversion) so the P.V product keeps ~16 bits of P.
// With A^1 written: two passes over the keys, (1) running row max / row sum,
// (2) recompute the scores, write A^1 rows and accumulate O. O-only (A^1 not
// written): one pass with an online softmax (running max, rescaled O and sum).
#include "pfa_kernels.h"
#include "pfa_split.h"

namespace pfa {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

constexpr int kDenseWaves = 8;
// O-only pass: how far (base 2) a tile's maximum may exceed the running reference
// point before the O rows are rescaled
constexpr float kStaleMax = 8.0f;

// max over lanes L and L ^ 16 (L ^ 32): a swap of 16-lane rows (32-lane halves)
// between two copies of x, no LDS round trip
__device__ __forceinline__ float max_xor16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
constexpr int kQPerBlock = 16 * kDenseWaves;

template <typename T, int D>
struct DenseOps;

// fp32: lane l covers dims [DPL*grp, DPL*grp + DPL) of its row, DPL = D/4, one
// MFMA step (k = 4: one dim per lane group) per dim of the run.
template <int D>
struct DenseOps<float, D> {
    static constexpr int DPL = D / 4;
    static constexpr int ROWB = D * 4;
    struct Row { float v[DPL]; };
    __device__ static Row load(const unsigned char* row, int grp) {
        Row r;
        const float* src = reinterpret_cast<const float*>(row) + grp * DPL;
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
    // P operand of the P.V product: the fp32 weights themselves
    struct PS { float p[4]; };
    __device__ static PS prep(const float p[4]) { return PS{{p[0], p[1], p[2], p[3]}}; }
    // V tile in LDS: KT rows of ROWB bytes, padded by 16
    template <int KT>
    static constexpr int vbuf() { return KT * (ROWB + 16); }
    template <int KT, int PER>
    __device__ static void store_v(unsigned char* dst, const uint4 (&reg)[PER]) {
        constexpr int CH = ROWB / 16;
#pragma unroll
        for (int x = 0; x < PER; ++x) {
            const int u = threadIdx.x + x * kDenseWaves * kWave;
            if (u < KT * CH) {
                const int t = u / CH;
                *reinterpret_cast<uint4*>(dst + t * (ROWB + 16) + (u - t * CH) * 16) = reg[x];
            }
        }
    }
    // O tile (16 queries x 16 dims) += P (16 q x 16 keys) . V (16 keys x 16 dims);
    // p[r]: weight of key key0 + r for query r16 (key0 = 16 s + 4 grp).
    template <int KT>
    __device__ static v4f pv(const PS& ps, const unsigned char* vt, int key0, int dim, v4f acc) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(
                ps.p[r], reinterpret_cast<const float*>(vt + (key0 + r) * (ROWB + 16))[dim], acc, 0, 0, 0);
        return acc;
    }
};

// bf16: lane l covers dims [DPL*grp, DPL*grp + DPL), DPL = D/4 (4 or 8), in MFMA
// steps of 4 bf16.
template <int D>
struct DenseOps<uint16_t, D> {
    static constexpr int DPL = D / 4;
    static constexpr int ROWB = D * 2;
    struct Row { v4s v[DPL / 4]; };
    __device__ static Row load(const unsigned char* row, int grp) {
        Row r;
        const uint16_t* src = reinterpret_cast<const uint16_t*>(row) + grp * DPL;
#pragma unroll
        for (int x = 0; x < DPL / 4; ++x) {
            // the 4 bf16 as they sit in memory (element e = bits 16e..16e+15)
            r.v[x] = __builtin_bit_cast(v4s, *reinterpret_cast<const uint2*>(src + 4 * x));
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
    // P split once per 16-key tile into bf16 hi + lo (round to nearest even with
    // v_cvt_pk_bf16_f32; the remainder is exact in fp32), ~16 bits of P in all
    // (values converted in pairs, so each conversion is one v_cvt_pk_bf16_f32 and the
    // packed hi words unpack with one shift or mask per value: 3 VALU per value)
    struct PS { v4s hi, lo; };
    __device__ static PS prep(const float p[4]) {
        const bf2 h01 = __builtin_convertvector(f2{p[0], p[1]}, bf2);
        const bf2 h23 = __builtin_convertvector(f2{p[2], p[3]}, bf2);
        const uint32_t u01 = __builtin_bit_cast(uint32_t, h01), u23 = __builtin_bit_cast(uint32_t, h23);
        const bf2 l01 = __builtin_convertvector(f2{p[0] - bf16_lo(u01), p[1] - bf16_hi(u01)}, bf2);
        const bf2 l23 = __builtin_convertvector(f2{p[2] - bf16_lo(u23), p[3] - bf16_hi(u23)}, bf2);
        PS ps;
        ps.hi = __builtin_bit_cast(v4s, make_uint2(u01, u23));
        ps.lo = __builtin_bit_cast(v4s, make_uint2(__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)));
        return ps;
    }
    // V tile in LDS transposed: D rows (dims) of KT keys, 8 bytes of padding, so the
    // B operand of the P.V MFMA (4 consecutive keys of one dim) is one 8-byte read
    template <int KT>
    static constexpr int vts() { return KT * 2 + 8; }
    template <int KT>
    static constexpr int vbuf() { return D * vts<KT>(); }
    template <int KT, int PER>
    __device__ static void store_v(unsigned char* dst, const uint4 (&reg)[PER]) {
        constexpr int CH = ROWB / 16;
#pragma unroll
        for (int x = 0; x < PER; ++x) {
            const int u = threadIdx.x + x * kDenseWaves * kWave;
            if (u < KT * CH) {
                const int t = u / CH;
                unsigned char* col = dst + (u - t * CH) * 8 * vts<KT>() + t * 2;   // dim 8c, key t
                const uint32_t wv[4] = {reg[x].x, reg[x].y, reg[x].z, reg[x].w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *reinterpret_cast<uint16_t*>(col + e * vts<KT>()) = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
            }
        }
    }
    template <int KT>
    __device__ static v4f pv(const PS& ps, const unsigned char* vt, int key0, int dim, v4f acc) {
        const v4s vv = *reinterpret_cast<const v4s*>(vt + dim * vts<KT>() + key0 * 2);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ps.hi, vv, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ps.lo, vv, acc, 0, 0, 0);
        return acc;
    }
};

// Copy rows [key0, key0 + KT) of a window (slot order) into an LDS tile with a
// padded row stride; one 16-byte chunk per thread and step.
template <int ROWB, int KT>
__device__ __forceinline__ void tile_load(uint4 (&reg)[(KT * ROWB / 16 + kDenseWaves * kWave - 1) /
                                                       (kDenseWaves * kWave)],
                                          const unsigned char* plane, const Geom& g, int wy, int wx, int key0) {
    constexpr int CH = ROWB / 16;
    constexpr int UNITS = KT * CH;
    constexpr int PER = (UNITS + kDenseWaves * kWave - 1) / (kDenseWaves * kWave);
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        const int u = threadIdx.x + x * kDenseWaves * kWave;
        if (u < UNITS) {
            const int t = u / CH;
            const int c = u - t * CH;
            reg[x] = *reinterpret_cast<const uint4*>(plane + (size_t)slot_pixel(g, wy, wx, key0 + t) * ROWB + c * 16);
        }
    }
}
template <int ROWB, int KT, int STRIDE>
__device__ __forceinline__ void tile_store(unsigned char* dst,
                                           const uint4 (&reg)[(KT * ROWB / 16 + kDenseWaves * kWave - 1) /
                                                              (kDenseWaves * kWave)]) {
    constexpr int CH = ROWB / 16;
    constexpr int UNITS = KT * CH;
    constexpr int PER = (UNITS + kDenseWaves * kWave - 1) / (kDenseWaves * kWave);
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        const int u = threadIdx.x + x * kDenseWaves * kWave;
        if (u < UNITS) {
            const int t = u / CH;
            const int c = u - t * CH;
            *reinterpret_cast<uint4*>(dst + t * STRIDE + c * 16) = reg[x];
        }
    }
}

// K tile of fp32 rows (d = 32) stored as three bf16 planes of KT rows x 80 bytes.
template <int KT>
__device__ __forceinline__ void tile_store_split(unsigned char* dst,
                                                 const uint4 (&reg)[(KT * 128 / 16 + kDenseWaves * kWave - 1) /
                                                                    (kDenseWaves * kWave)]) {
    constexpr int CH = 8;
    constexpr int UNITS = KT * CH;
    constexpr int PER = (UNITS + kDenseWaves * kWave - 1) / (kDenseWaves * kWave);
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        const int u = threadIdx.x + x * kDenseWaves * kWave;
        if (u < UNITS) {
            const int t = u / CH;
            const int c = u - t * CH;
            const float f[4] = {__uint_as_float(reg[x].x), __uint_as_float(reg[x].y), __uint_as_float(reg[x].z),
                                __uint_as_float(reg[x].w)};
            bf4 h, m, l;
            split3<4>(f, h, m, l);
            unsigned char* row = dst + t * kSplitRow + c * 8;
            *reinterpret_cast<bf4*>(row) = h;
            *reinterpret_cast<bf4*>(row + KT * kSplitRow) = m;
            *reinterpret_cast<bf4*>(row + 2 * KT * kSplitRow) = l;
        }
    }
}

// BIAS: the head's relative position bias (a (2w - 1)^2 table, staged in LDS
// in base-2 units) is added to every scaled score; needs win % 16 == 0 so that
// the 16 keys of an MFMA tile share one window row.
template <typename T, int D, int KT, bool WA, bool BIAS = false>
__global__ __launch_bounds__(kDenseWaves * kWave) void dense_layer_kernel(const DenseArgs p) {
    using Ops = DenseOps<T, D>;
    constexpr int ROWB = Ops::ROWB;
    constexpr int STRIDE = ROWB + 16;             // padded LDS row
    constexpr int SUB = KT / 16;                   // 16-key MFMA tiles per LDS tile
    constexpr int CT = D / 16;                     // 16-dim output tiles
    constexpr int PER = (KT * ROWB / 16 + kDenseWaves * kWave - 1) / (kDenseWaves * kWave);
    // fp32, d = 32, 64-key tiles: scores from the three-way bf16 split
    constexpr bool SPLIT = sizeof(T) == 4 && D == 32 && KT == 64;
    constexpr int KBUF = SPLIT ? 3 * KT * kSplitRow : KT * STRIDE;
    __shared__ __align__(16) unsigned char Ks[2][KBUF];
    __shared__ __align__(16) unsigned char Vs[2][Ops::template vbuf<KT>()];
    __shared__ float btab[BIAS ? 63 * 63 : 1];

    const Geom g = p.g;
    const int N = g.N;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    const int qblocks = (N + kQPerBlock - 1) / kQPerBlock;
    int wh, qb;
    if (p.xcd_map) {   // the query blocks of one window-head are consecutive workgroups of one XCD
        const int xcd = blockIdx.x & 7;
        const int slot = blockIdx.x >> 3;
        qb = slot % qblocks;
        wh = (slot / qblocks) * 8 + xcd;
    } else {
        wh = blockIdx.x / qblocks;
        qb = blockIdx.x - wh * qblocks;
    }
    const int q0 = qb * kQPerBlock + wave * 16;
    const bool wave_active = q0 < N;   // idle waves still take part in the tile barriers
    const int nwin = g.nwy * g.nwx;
    const int win_id = wh % nwin;
    const int bh = wh / nwin;
    const int wy = win_id / g.nwx;
    const int wx = win_id - wy * g.nwx;
    const size_t plane = (size_t)bh * g.H * g.W * D;
    const unsigned char* Qh = reinterpret_cast<const unsigned char*>(static_cast<const T*>(p.Q) + plane);
    const unsigned char* Kh = reinterpret_cast<const unsigned char*>(static_cast<const T*>(p.K) + plane);
    const unsigned char* Vh = reinterpret_cast<const unsigned char*>(static_cast<const T*>(p.V) + plane);
    float* Oh = p.O_out + plane;
    const float sc = p.scale2;

    // bias: this lane's query i = q0 + r16 at window row/column (iy, ix); key j
    // of a tile at (jy, jx) reads btab[ibase - jy (2w - 1) - jx]
    int ibase = 0;
    const int wrow = 2 * g.win - 1;
    if constexpr (BIAS) {
        const int nrel = wrow * wrow;
        const float* src = p.bias + (size_t)(bh % g.heads) * nrel;
        for (int u = threadIdx.x; u < nrel; u += blockDim.x) btab[u] = src[u] * 1.4426950408889634f;
        const int i = wave_active ? q0 + r16 : 0;
        const int iy = i / g.win;
        ibase = (iy + g.win - 1) * wrow + (i - iy * g.win) + g.win - 1;
    }
    // bias of keys key0 + 4 grp + r, r = 0..3 (one window row)
    auto tile_bias = [&](int key0, float (&b)[4]) {
        const int jy = key0 / g.win;
        const int idx0 = ibase - jy * wrow - (key0 - jy * g.win) - 4 * grp;
#pragma unroll
        for (int r = 0; r < 4; ++r) b[r] = btab[idx0 - r];
    };
    const int qrow = wave_active ? q0 + r16 : 0;
    const typename Ops::Row qop = Ops::load(Qh + (size_t)slot_pixel(g, wy, wx, qrow) * ROWB, grp);
    bf8 qh, qm, ql;   // SPLIT: lane's 8 dims of its query in three parts
    if constexpr (SPLIT) split3<8>(reinterpret_cast<const float*>(&qop), qh, qm, ql);
    // 16 keys x 16 queries of scores from LDS tile kt, subtile s
    auto tile_scores = [&](const unsigned char* kt, int s) -> v4f {
        if constexpr (SPLIT) {
            const unsigned char* row = kt + (s * 16 + r16) * kSplitRow + grp * 16;
            const bf8 kh = *reinterpret_cast<const bf8*>(row);
            const bf8 km = *reinterpret_cast<const bf8*>(row + KT * kSplitRow);
            const bf8 kl = *reinterpret_cast<const bf8*>(row + 2 * KT * kSplitRow);
            return dot_split3(kh, km, kl, qh, qm, ql, v4f{0.f, 0.f, 0.f, 0.f});
        } else {
            const typename Ops::Row kop = Ops::load(kt + (s * 16 + r16) * STRIDE, grp);
            return Ops::scores(kop, qop);
        }
    };
    auto store_k = [&](unsigned char* dst, const uint4 (&reg)[PER]) {
        if constexpr (SPLIT) tile_store_split<KT>(dst, reg);
        else tile_store<ROWB, KT, STRIDE>(dst, reg);
    };
    const int ntiles = N / KT;
    uint4 kreg[PER], vreg[PER];
    uint4 kreg2[PER], vreg2[PER];   // the second register set (odd tiles)

    if constexpr (!WA) {
        // O-only: one pass with an online softmax. Per K/V tile, the running max m
        // of the lane's query (shared by its 4 lane groups) is raised to the tile's
        // maximum; the O rows and the partial sums are rescaled by 2^(m_old - m)
        // (an O accumulator row is another query's: its factor comes from the lane
        // that owns that query), then P = 2^(s - m) is accumulated into O = P V.
        float m = -INFINITY, l = 0.0f;
        v4f oacc[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) oacc[c] = v4f{0.f, 0.f, 0.f, 0.f};
        tile_load<ROWB, KT>(kreg, Kh, g, wy, wx, 0);
        tile_load<ROWB, KT>(vreg, Vh, g, wy, wx, 0);
        store_k(Ks[0], kreg);
        Ops::template store_v<KT>(Vs[0], vreg);
        if (ntiles > 1) {
            tile_load<ROWB, KT>(kreg2, Kh, g, wy, wx, KT);
            tile_load<ROWB, KT>(vreg2, Vh, g, wy, wx, KT);
        }
        __syncthreads();
        auto step = [&](int t, uint4 (&kld)[PER], uint4 (&vld)[PER], const uint4 (&kst)[PER],
                        const uint4 (&vst)[PER]) {
            if (t + 2 < ntiles) {
                tile_load<ROWB, KT>(kld, Kh, g, wy, wx, (t + 2) * KT);
                tile_load<ROWB, KT>(vld, Vh, g, wy, wx, (t + 2) * KT);
            }
            const unsigned char* kt = Ks[t & 1];
            const unsigned char* vt = Vs[t & 1];
            v4f acc[SUB];
#pragma unroll
            for (int s = 0; s < SUB; ++s) acc[s] = tile_scores(kt, s);
            // scaled and biased scores in base-2 units; without a bias the scores stay
            // raw and the scale is folded into the exponent's argument below (the row
            // maximum scales with them: rounding of x * sc is monotone for sc > 0)
            if constexpr (BIAS) {
#pragma unroll
                for (int s = 0; s < SUB; ++s) {
                    float b[4] = {0.f, 0.f, 0.f, 0.f};
                    tile_bias(t * KT + s * 16, b);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[s][r] = fmaf(acc[s][r], sc, b[r]);
                }
            }
            float tmax = acc[0][0];
#pragma unroll
            for (int s = 0; s < SUB; ++s)
#pragma unroll
                for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, acc[s][r]);
            tmax = max_xor16(tmax);
            tmax = max_xor32(tmax);
            if constexpr (!BIAS) tmax *= sc;
            // The reference point m moves only when a tile's maximum exceeds it by more
            // than kStaleMax (base-2 units), so P stays below 2^kStaleMax and the O
            // rows are rescaled only on those tiles (the first one, and rarely later).
            // Any m works: it cancels between O and l.
            const bool grow = tmax > m + kStaleMax;   // the 4 lane groups of a query agree
            if (ballot(grow) != 0) {
                const float mn = grow ? tmax : m;
                const float alpha = fast_exp2(m - mn);   // 0 on the first tile (m = -inf)
                m = mn;
                l *= alpha;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ar = __shfl(alpha, 4 * grp + r);   // factor of O row 4 grp + r
#pragma unroll
                    for (int c = 0; c < CT; ++c) oacc[c][r] *= ar;
                }
            }
#pragma unroll
            for (int s = 0; s < SUB; ++s) {
                float pr[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pr[r] = BIAS ? fast_exp2(acc[s][r] - m) : fast_exp2(fmaf(acc[s][r], sc, -m));
                    l += pr[r];
                }
                const typename Ops::PS ps = Ops::prep(pr);
#pragma unroll
                for (int c = 0; c < CT; ++c)
                    oacc[c] = Ops::template pv<KT>(ps, vt, s * 16 + 4 * grp, c * 16 + r16, oacc[c]);
            }
            if (t + 1 < ntiles) {
                store_k(Ks[(t + 1) & 1], kst);
                Ops::template store_v<KT>(Vs[(t + 1) & 1], vst);
            }
            __syncthreads();
        };
        for (int t = 0; t < ntiles; t += 2) {
            step(t, kreg, vreg, kreg2, vreg2);
            if (t + 1 < ntiles) step(t + 1, kreg2, vreg2, kreg, vreg);
        }
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (p.lse_out && wave_active && grp == 0 && q0 + r16 < N)
            p.lse_out[(size_t)wh * N + q0 + r16] = (m + __builtin_amdgcn_logf(l)) * 0.6931471805599453f;
        if (!wave_active) return;
        const float inv_l = 1.0f / l;
        // lane holds O[query q0 + 4*grp + r][dim 16c + r16]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float ir = __shfl(inv_l, 4 * grp + r);
            float* orow = Oh + (size_t)slot_pixel(g, wy, wx, q0 + 4 * grp + r) * D;
#pragma unroll
            for (int c = 0; c < CT; ++c) orow[c * 16 + r16] = oacc[c][r] * ir;
        }
        return;
    }

    // pass 1: per-lane running max / sum over the keys 4*grp + r of every 16-key tile
    float m = -INFINITY, l = 0.0f;
    tile_load<ROWB, KT>(kreg, Kh, g, wy, wx, 0);
    store_k(Ks[0], kreg);
    if (ntiles > 1) tile_load<ROWB, KT>(kreg2, Kh, g, wy, wx, KT);
    __syncthreads();
    // ld: the registers of tile t (already in LDS), refilled with tile t + 2; st: tile t + 1
    auto pass1 = [&](int t, uint4 (&ld)[PER], const uint4 (&st)[PER]) {
        if (t + 2 < ntiles) tile_load<ROWB, KT>(ld, Kh, g, wy, wx, (t + 2) * KT);
        const unsigned char* kt = Ks[t & 1];
        // the whole tile's scores, then one rescale of the running sum (m is in
        // scaled base-2 units; sc > 0, so the raw maximum gives the scaled one)
        v4f acc[SUB];
#pragma unroll
        for (int s = 0; s < SUB; ++s) acc[s] = tile_scores(kt, s);
        float lt = 0.0f;
        float mn;
        if constexpr (BIAS) {
            // biased scores in scaled units, then the same running max / sum
#pragma unroll
            for (int s = 0; s < SUB; ++s) {
                float b[4];
                tile_bias(t * KT + s * 16, b);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[s][r] = fmaf(acc[s][r], sc, b[r]);
            }
            float amax = acc[0][0];
#pragma unroll
            for (int s = 0; s < SUB; ++s)
#pragma unroll
                for (int r = 0; r < 4; ++r) amax = fmaxf(amax, acc[s][r]);
            mn = fmaxf(m, amax);
#pragma unroll
            for (int s = 0; s < SUB; ++s)
#pragma unroll
                for (int r = 0; r < 4; ++r) lt += fast_exp2(acc[s][r] - mn);
        } else {
            float amax = acc[0][0];
#pragma unroll
            for (int s = 0; s < SUB; ++s)
#pragma unroll
                for (int r = 0; r < 4; ++r) amax = fmaxf(amax, acc[s][r]);
            mn = fmaxf(m, amax * sc);
#pragma unroll
            for (int s = 0; s < SUB; ++s)
#pragma unroll
                for (int r = 0; r < 4; ++r) lt += fast_exp2(fmaf(acc[s][r], sc, -mn));
        }
        l = l * fast_exp2(m - mn) + lt;
        m = mn;
        if (t + 1 < ntiles) store_k(Ks[(t + 1) & 1], st);
        __syncthreads();
    };
    for (int t = 0; t < ntiles; t += 2) {
        pass1(t, kreg, kreg2);
        if (t + 1 < ntiles) pass1(t + 1, kreg2, kreg);
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
    // ln of the softmax denominator: sum_j exp(s_ij) = 2^m * l with s in natural units
    if (p.lse_out && wave_active && grp == 0 && q0 + r16 < N)
        p.lse_out[(size_t)wh * N + q0 + r16] = (m + __builtin_amdgcn_logf(l)) * 0.6931471805599453f;

    // pass 2: probabilities, A^1 rows, O += P V
    v4f oacc[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) oacc[c] = v4f{0.f, 0.f, 0.f, 0.f};
    // A^1 rows of the wave's 16 queries through a buffer resource (an empty range
    // for an idle wave, so its stores are dropped)
    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc(WA ? p.A_out + ((size_t)wh * N + (wave_active ? q0 : 0)) * N : nullptr,
                  (WA && wave_active) ? 16 * N * 4 : 0);
    tile_load<ROWB, KT>(kreg, Kh, g, wy, wx, 0);
    tile_load<ROWB, KT>(vreg, Vh, g, wy, wx, 0);
    store_k(Ks[0], kreg);
    Ops::template store_v<KT>(Vs[0], vreg);
    if (ntiles > 1) {
        tile_load<ROWB, KT>(kreg2, Kh, g, wy, wx, KT);
        tile_load<ROWB, KT>(vreg2, Vh, g, wy, wx, KT);
    }
    __syncthreads();
    auto pass2 = [&](int t, uint4 (&kld)[PER], uint4 (&vld)[PER], const uint4 (&kst)[PER],
                     const uint4 (&vst)[PER]) {
        if (t + 2 < ntiles) {
            tile_load<ROWB, KT>(kld, Kh, g, wy, wx, (t + 2) * KT);
            tile_load<ROWB, KT>(vld, Vh, g, wy, wx, (t + 2) * KT);
        }
        const unsigned char* kt = Ks[t & 1];
        const unsigned char* vt = Vs[t & 1];
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
            const v4f acc = tile_scores(kt, s);
            float pr[4];
            if constexpr (BIAS) {
                float b[4];
                tile_bias(t * KT + s * 16, b);
#pragma unroll
                for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(fmaf(acc[r], sc, b[r] - m)) * inv_l;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(fmaf(acc[r], sc, -m)) * inv_l;
            }
            if (WA) {
                typedef int v4i __attribute__((ext_vector_type(4)));
                const v4i pv = {__float_as_int(pr[0]), __float_as_int(pr[1]), __float_as_int(pr[2]),
                                __float_as_int(pr[3])};
                __builtin_amdgcn_raw_buffer_store_b128(pv, rA, (r16 * N + t * KT + s * 16 + 4 * grp) * 4, 0, 0);
            }
            const typename Ops::PS ps = Ops::prep(pr);
#pragma unroll
            for (int c = 0; c < CT; ++c)
                oacc[c] = Ops::template pv<KT>(ps, vt, s * 16 + 4 * grp, c * 16 + r16, oacc[c]);
        }
        if (t + 1 < ntiles) {
            store_k(Ks[(t + 1) & 1], kst);
            Ops::template store_v<KT>(Vs[(t + 1) & 1], vst);
        }
        __syncthreads();
    };
    for (int t = 0; t < ntiles; t += 2) {
        pass2(t, kreg, vreg, kreg2, vreg2);
        if (t + 1 < ntiles) pass2(t + 1, kreg2, vreg2, kreg, vreg);
    }
    if (!wave_active) return;
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

template <typename T, int D, bool WA>
void launch_dense_w(const DenseArgs& a, int grid, hipStream_t s) {
    if (a.bias) {   // win % 16 == 0 (checked by the caller)
        if (a.g.N % 64 == 0)
            hipLaunchKernelGGL((dense_layer_kernel<T, D, 64, WA, true>), dim3(grid), dim3(kDenseWaves * kWave), 0, s,
                               a);
        else
            hipLaunchKernelGGL((dense_layer_kernel<T, D, 16, WA, true>), dim3(grid), dim3(kDenseWaves * kWave), 0, s,
                               a);
        return;
    }
    if (a.g.N % 64 == 0)
        hipLaunchKernelGGL((dense_layer_kernel<T, D, 64, WA>), dim3(grid), dim3(kDenseWaves * kWave), 0, s, a);
    else
        hipLaunchKernelGGL((dense_layer_kernel<T, D, 16, WA>), dim3(grid), dim3(kDenseWaves * kWave), 0, s, a);
}

template <typename T, int D>
void launch_dense_t(const DenseArgs& a, int grid, hipStream_t s) {
    if (a.A_out) launch_dense_w<T, D, true>(a, grid, s);
    else launch_dense_w<T, D, false>(a, grid, s);
}

}  // namespace

int dense_query_blocks(int N) { return (N + kQPerBlock - 1) / kQPerBlock; }

hipError_t launch_dense(const DenseArgs& a, int dtype, int D, int grid, hipStream_t stream) {
    if (dtype == 0) {
        if (D == 16) launch_dense_t<float, 16>(a, grid, stream);
        else launch_dense_t<float, 32>(a, grid, stream);
    } else {
        if (D == 16) launch_dense_t<uint16_t, 16>(a, grid, stream);
        else launch_dense_t<uint16_t, 32>(a, grid, stream);
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
