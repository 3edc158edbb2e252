// Backward pass of the dense first layer on gfx950 (matrix cores).
//
// The first layer is softmax attention over the N slots of a window (paper notes
// "Progressive Focused Transformer for Single Image Super-Resolution", section
// "Progressive focused resource allocation strategy"): P_ij = exp(s_ij - lse_i),
// s_ij = q_i.k_j / sqrt(d) (+ the relative position bias), O = P V. Its map A^1 = P
// also feeds the second layer, so the gradient of the loss reaches it both
// through O and directly (dA = the second layer's gradient of A^{l-1}):
//   G_ij = dA_ij + dO_i.v_j,   D_i = sum_j P_ij G_ij,   dS_ij = P_ij (G_ij - D_i)
//   dQ = dS K / sqrt(d),   dK = dS^T Q / sqrt(d),   dV = P^T dO.
// P is recomputed from Q, K and the forward's log denominators lse (what the
// dense layer writes to lse_out).
//
// dense_bwd_dq_kernel: 8 waves x 16 queries per workgroup; K/V tiles of 64 slots
//   staged in LDS, double-buffered (the loads of the tile after next in flight). Pass 1
//   accumulates D_i, pass 2 forms dS and dQ. Scores and dO.v come transposed
//   (16 keys x 16 queries per tile), which leaves lane (query r16, keys
//   4 grp + r): the A-operand layout of dS K (v_mfma_f32_16x16x4_f32).
// dense_bwd_dkv_kernel: 8 waves x 16 keys per workgroup; Q/dO tiles of 64 slots
//   (with their lse and D) staged in LDS. Scores as (query 4 grp + r, key r16)
//   per lane: the A-operand layout of P^T dO and dS^T Q (fp32 MFMA). dV, dK stay
//   in registers over all query tiles.
// With d = 32 and no bias both kernels compute the scores and dO.v on
// v_mfma_f32_16x16x32_bf16 from the three-way bf16 split of their fp32 operands
// (as accurate as fp32 products; pfa_split.h), the tile side split once per tile
// into bf16 planes in LDS; otherwise on v_mfma_f32_16x16x4_f32.
#include "pfa_kernels.h"
#include "pfa_rows.h"
#include "pfa_split.h"

namespace pfa {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBwdWaves = 8;
constexpr int kTile = 64;          // slots per LDS tile
constexpr float kLog2e = 1.4426950408889634f;

// Tiles of rows [r0, r0 + kTile) of a window (slot order): loaded from global
// memory into registers (16-byte chunks, one or more per thread), then written
// to LDS as fp32 with a row stride of STR floats. Splitting the two steps lets
// the next tile's loads be in flight while the current tile is used.
template <typename T, int D>
struct TileRegs {
    static constexpr int EPC = Chunk<T>::kElems;
    static constexpr int CH = D / EPC;
    static constexpr int UNITS = kTile * CH;
    static constexpr int PER = (UNITS + kBwdWaves * kWave - 1) / (kBwdWaves * kWave);
    uint4 r[PER];
    __device__ void load(const T* plane, const Geom& g, int wy, int wx, int r0) {
#pragma unroll
        for (int x = 0; x < PER; ++x) {
            const int u = threadIdx.x + x * kBwdWaves * kWave;
            if (u < UNITS) {
                const int t = u / CH;
                const int c = u - t * CH;
                r[x] = *reinterpret_cast<const uint4*>(reinterpret_cast<const unsigned char*>(plane) +
                                                       ((size_t)slot_pixel(g, wy, wx, r0 + t) * D) * sizeof(T) +
                                                       c * 16);
            }
        }
    }
    template <int STR>
    __device__ void store(float* dst) const {
#pragma unroll
        for (int x = 0; x < PER; ++x) {
            const int u = threadIdx.x + x * kBwdWaves * kWave;
            if (u < UNITS) {
                const int t = u / CH;
                const int c = u - t * CH;
                float f[EPC];
                Chunk<T>::to_f32(r[x], f);
#pragma unroll
                for (int e = 0; e < EPC; e += 4)
                    *reinterpret_cast<float4*>(dst + t * STR + c * EPC + e) = make_float4(f[e], f[e + 1], f[e + 2],
                                                                                         f[e + 3]);
            }
        }
    }
    // d = 32: the tile as bf16 planes of kTile rows x 64 bytes, 16-byte chunk m of
    // row t stored at chunk position m ^ ((t >> 2) & 3), so the operand reads of 16
    // consecutive rows at one chunk hit distinct banks; fp32 rows as three planes
    // (hi, mid, lo), bf16 rows (exact) as one
    __device__ void store_planes64(unsigned char* dst) const {
        static_assert(D == 32, "planes hold 32-wide rows");
#pragma unroll
        for (int x = 0; x < PER; ++x) {
            const int u = threadIdx.x + x * kBwdWaves * kWave;
            if (u < UNITS) {
                const int t = u / CH;
                const int c = u - t * CH;
                if constexpr (sizeof(T) == 4) {   // chunk c = dims 4c .. 4c + 3: half of a bf16 chunk
                    const float f[4] = {__uint_as_float(r[x].x), __uint_as_float(r[x].y), __uint_as_float(r[x].z),
                                        __uint_as_float(r[x].w)};
                    bf4 h, m, l;
                    split3<4>(f, h, m, l);
                    unsigned char* row = dst + t * 64 + (((c >> 1) ^ ((t >> 2) & 3)) << 4) + (c & 1) * 8;
                    *reinterpret_cast<bf4*>(row) = h;
                    *reinterpret_cast<bf4*>(row + kTile * 64) = m;
                    *reinterpret_cast<bf4*>(row + 2 * kTile * 64) = l;
                } else {   // chunk c = dims 8c .. 8c + 7
                    *reinterpret_cast<uint4*>(dst + t * 64 + ((c ^ ((t >> 2) & 3)) << 4)) = r[x];
                }
            }
        }
    }
    // d = 32: the tile as bf16 planes of kTile rows x kSplitRow bytes; fp32 rows as
    // three planes (hi, mid, lo), bf16 rows (exact) as one
    __device__ void store_planes(unsigned char* dst) const {
        static_assert(D == 32, "planes hold 32-wide rows");
#pragma unroll
        for (int x = 0; x < PER; ++x) {
            const int u = threadIdx.x + x * kBwdWaves * kWave;
            if (u < UNITS) {
                const int t = u / CH;
                const int c = u - t * CH;
                if constexpr (sizeof(T) == 4) {
                    const float f[4] = {__uint_as_float(r[x].x), __uint_as_float(r[x].y), __uint_as_float(r[x].z),
                                        __uint_as_float(r[x].w)};
                    bf4 h, m, l;
                    split3<4>(f, h, m, l);
                    unsigned char* row = dst + t * kSplitRow + c * 8;
                    *reinterpret_cast<bf4*>(row) = h;
                    *reinterpret_cast<bf4*>(row + kTile * kSplitRow) = m;
                    *reinterpret_cast<bf4*>(row + 2 * kTile * kSplitRow) = l;
                } else {
                    *reinterpret_cast<uint4*>(dst + t * kSplitRow + c * 16) = r[x];
                }
            }
        }
    }
};

// this lane's DPL dims [DPL grp, DPL grp + DPL) of one row of a [.., D] array of type T
template <typename T, int D>
__device__ __forceinline__ void row_dims(const T* row, int grp, float (&o)[D / 4]) {
    constexpr int DPL = D / 4;
    if constexpr (sizeof(T) == 4) {
        const float* src = reinterpret_cast<const float*>(row) + grp * DPL;
#pragma unroll
        for (int x = 0; x < DPL; x += 4) {
            const float4 f = *reinterpret_cast<const float4*>(src + x);
            o[x] = f.x; o[x + 1] = f.y; o[x + 2] = f.z; o[x + 3] = f.w;
        }
    } else {
        const uint16_t* src = reinterpret_cast<const uint16_t*>(row) + grp * DPL;
#pragma unroll
        for (int x = 0; x < DPL; ++x) o[x] = __uint_as_float((uint32_t)src[x] << 16);
    }
}

struct BlockPos {
    int wh, blk, wy, wx, bh;
};
__device__ __forceinline__ BlockPos decode(const Geom& g, int blocks, int xcd_map) {
    BlockPos b;
    if (xcd_map) {   // the blocks of one window-head are consecutive workgroups of one XCD
        const int xcd = blockIdx.x & 7;
        const int slot = blockIdx.x >> 3;
        b.blk = slot % blocks;
        b.wh = (slot / blocks) * 8 + xcd;
    } else {
        b.wh = blockIdx.x / blocks;
        b.blk = blockIdx.x - b.wh * blocks;
    }
    const int nwin = g.nwy * g.nwx;
    const int win_id = b.wh % nwin;
    b.bh = b.wh / nwin;
    b.wy = win_id / g.nwx;
    b.wx = win_id - b.wy * g.nwx;
    return b;
}

template <typename T, int D, bool BIAS, bool HAS_DA, bool DBIAS>
__global__ __launch_bounds__(kBwdWaves * kWave) void dense_bwd_dq_kernel(const DenseBwdArgs p) {
    static_assert(!DBIAS || BIAS, "the bias gradient comes with a bias");
    constexpr int DPL = D / 4;
    constexpr int CT = D / 16;
    constexpr int STR = D + 4;   // padded fp32 LDS row
    constexpr int SUB = kTile / 16;
    // SPLIT (d = 32, no bias): scores and dO.v on bf16 MFMA from bf16 planes of the
    // K/V tiles (three-way split of fp32 values; bf16 inputs are exact as they are)
    constexpr bool SPLIT = D == 32 && !BIAS;
    constexpr bool BFIN = sizeof(T) == 2;
    constexpr int PLB = SPLIT ? (BFIN ? 1 : 3) * kTile * kSplitRow : 16;
    __shared__ __align__(16) float Kt2[2][kTile * STR];
    __shared__ __align__(16) float Vt2[SPLIT ? 1 : 2][SPLIT ? 4 : kTile * STR];
    __shared__ __align__(16) unsigned char KP2[SPLIT ? 2 : 1][PLB];
    __shared__ __align__(16) unsigned char VP2[SPLIT ? 2 : 1][PLB];
    __shared__ float btab[BIAS ? 63 * 63 : 1];
    // DBIAS: each wave's 16 x 16 block of dS, row stride 20 floats (16-byte aligned rows)
    __shared__ __align__(16) float dtile[DBIAS ? kBwdWaves * 16 * 20 : 4];

    const Geom g = p.g;
    const int N = g.N;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    const BlockPos bp = decode(g, (N + 16 * kBwdWaves - 1) / (16 * kBwdWaves), p.xcd_map);
    const int q0 = bp.blk * 16 * kBwdWaves + wave * 16;
    const bool wave_active = q0 < N;
    const size_t plane = (size_t)bp.bh * g.H * g.W * D;
    const T* Qh = static_cast<const T*>(p.Q) + plane;
    const T* Kh = static_cast<const T*>(p.K) + plane;
    const T* Vh = static_cast<const T*>(p.V) + plane;
    const float sc = p.scale2;

    const int qi = wave_active ? q0 + r16 : 0;   // this lane's query (operand layout)
    float qv[DPL], dov[DPL];
    row_dims<T, D>(Qh + (size_t)slot_pixel(g, bp.wy, bp.wx, qi) * D, grp, qv);
    row_dims<float, D>(p.dO + plane + (size_t)slot_pixel(g, bp.wy, bp.wx, qi) * D, grp, dov);
    const float lse2 = p.lse[(size_t)bp.wh * N + qi] * kLog2e;
    bf8 qh, qm, ql, dh, dm, dl;   // SPLIT: this lane's 8 dims of q and dO in parts
    if constexpr (SPLIT) {
        split3<8>(qv, qh, qm, ql);
        split3<8>(dov, dh, dm, dl);
    }
    const int wrow = 2 * g.win - 1;
    int ibase = 0;
    if constexpr (BIAS) {
        const int nrel = wrow * wrow;
        const float* src = p.bias + (size_t)(bp.bh % g.heads) * nrel;
        for (int u = threadIdx.x; u < nrel; u += blockDim.x) btab[u] = src[u] * kLog2e;
        const int iy = qi / g.win;
        ibase = (iy + g.win - 1) * wrow + (qi - iy * g.win) + g.win - 1;
    }
    const float* dArow = HAS_DA ? p.dA + ((size_t)bp.wh * N + qi) * N : nullptr;

    float Dq = 0.0f;
    // DBIAS: lane L sums dS over the pairs of this wave's queries at horizontal offset
    // dx = L - (win - 1) and the vertical offset of the current key row (flushed per row)
    float dacc = 0.0f;
    v4f dq[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) dq[c] = v4f{0.f, 0.f, 0.f, 0.f};
    // the tile sequence of both passes: LDS double-buffered, the global loads two
    // tiles ahead in two register sets (tile it + 2 is loaded while tile it is used
    // from LDS and tile it + 1 waits in registers)
    const int ntiles = N / kTile;
    TileRegs<T, D> kreg, vreg, kreg2, vreg2;
    auto store_tiles = [&](int b, const TileRegs<T, D>& kr, const TileRegs<T, D>& vr) {
        kr.template store<STR>(Kt2[b]);
        if constexpr (SPLIT) {
            kr.store_planes(KP2[b]);
            vr.store_planes(VP2[b]);
        } else {
            vr.template store<STR>(Vt2[b]);
        }
    };
    kreg.load(Kh, g, bp.wy, bp.wx, 0);
    vreg.load(Vh, g, bp.wy, bp.wx, 0);
    store_tiles(0, kreg, vreg);
    {
        const int t1 = (1 % ntiles) * kTile;
        kreg2.load(Kh, g, bp.wy, bp.wx, t1);
        vreg2.load(Vh, g, bp.wy, bp.wx, t1);
    }
    __syncthreads();
    auto step = [&](int it, TileRegs<T, D>& kld, TileRegs<T, D>& vld, const TileRegs<T, D>& kst,
                    const TileRegs<T, D>& vst) {
        const int pass = it / ntiles;
        const int t0 = (it - pass * ntiles) * kTile;
        const float* Kt = Kt2[it & 1];
        const float* Vt = Vt2[SPLIT ? 0 : (it & 1)];
        // this tile's dA^1 (4 keys per lane and 16-key step) before the next tile's
        // loads: waits count loads in issue order, so the prefetch stays in flight
        float4 dat[SUB];
#pragma unroll
        for (int s = 0; s < SUB; ++s)
            dat[s] = HAS_DA ? *reinterpret_cast<const float4*>(dArow + t0 + s * 16 + 4 * grp)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
        if (it + 2 < 2 * ntiles) {
            const int tn = ((it + 2) % ntiles) * kTile;
            kld.load(Kh, g, bp.wy, bp.wx, tn);
            vld.load(Vh, g, bp.wy, bp.wx, tn);
        }
        {
#pragma unroll
            for (int s = 0; s < SUB; ++s) {
                const int key0 = t0 + s * 16;
                v4f st = {0.f, 0.f, 0.f, 0.f}, dpt = {0.f, 0.f, 0.f, 0.f};
                if constexpr (SPLIT) {
                    // A rows: keys s*16 + r16, dims 8 grp .. 8 grp + 7 of each plane
                    const unsigned char* kp = KP2[it & 1] + (s * 16 + r16) * kSplitRow + grp * 16;
                    const unsigned char* vp = VP2[it & 1] + (s * 16 + r16) * kSplitRow + grp * 16;
                    const bf8 kh = *reinterpret_cast<const bf8*>(kp);
                    const bf8 vh = *reinterpret_cast<const bf8*>(vp);
                    if constexpr (BFIN) {   // k, q, v exact in bf16: one product each, dO in three parts
                        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh, st, 0, 0, 0);
                        dpt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vh, dl, dpt, 0, 0, 0);
                        dpt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vh, dm, dpt, 0, 0, 0);
                        dpt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vh, dh, dpt, 0, 0, 0);
                    } else {
                        const bf8 km = *reinterpret_cast<const bf8*>(kp + kTile * kSplitRow);
                        const bf8 kl = *reinterpret_cast<const bf8*>(kp + 2 * kTile * kSplitRow);
                        const bf8 vm = *reinterpret_cast<const bf8*>(vp + kTile * kSplitRow);
                        const bf8 vl = *reinterpret_cast<const bf8*>(vp + 2 * kTile * kSplitRow);
                        st = dot_split3(kh, km, kl, qh, qm, ql, st);
                        dpt = dot_split3(vh, vm, vl, dh, dm, dl, dpt);
                    }
                } else {
                    const float* kr = Kt + (s * 16 + r16) * STR + DPL * grp;
                    const float* vr = Vt + (s * 16 + r16) * STR + DPL * grp;
#pragma unroll
                    for (int x = 0; x < DPL; ++x) {
                        st = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[x], qv[x], st, 0, 0, 0);
                        dpt = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[x], dov[x], dpt, 0, 0, 0);
                    }
                }
                // lane: query qi, keys key0 + 4 grp + r
                float b[4] = {0.f, 0.f, 0.f, 0.f};
                if constexpr (BIAS) {
                    const int jy = key0 / g.win;
                    const int idx0 = ibase - jy * wrow - (key0 - jy * g.win) - 4 * grp;
#pragma unroll
                    for (int r = 0; r < 4; ++r) b[r] = btab[idx0 - r];
                }
                const float dav[4] = {dat[s].x, dat[s].y, dat[s].z, dat[s].w};
                float P[4], G[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    P[r] = fast_exp2(fmaf(st[r], sc, b[r] - lse2));
                    G[r] = dpt[r] + dav[r];
                }
                if (pass == 0) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) Dq = fmaf(P[r], G[r], Dq);
                } else {
                    float dS[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) dS[r] = P[r] * (G[r] - Dq);
                    if constexpr (DBIAS) {
                        // the block's queries (one window row, columns qx0 + r16) and keys (one
                        // window row, columns kx0 + c) pair at column offset qx0 - kx0 + (r16 - c):
                        // diagonal m = r16 - c of the block. The wave's own LDS writes and reads
                        // complete in issue order, so no barrier is needed.
                        float* Tw = dtile + wave * (16 * 20);
                        *reinterpret_cast<float4*>(Tw + r16 * 20 + 4 * grp) = make_float4(dS[0], dS[1], dS[2], dS[3]);
                        const int jy = key0 / g.win;
                        const int kx0 = key0 - jy * g.win;
                        const int m = lane - (g.win - 1) - (q0 - (q0 / g.win) * g.win - kx0);
                        if (m >= -15 && m <= 15) {
                            const int qa = m > 0 ? m : 0;
                            const int qb = m < 0 ? 15 + m : 15;
                            float dsum = 0.0f;
                            for (int q = qa; q <= qb; ++q) dsum += Tw[q * 21 - m];
                            dacc += dsum;
                        }
                        if (kx0 + 16 == g.win) {   // the key row is complete
                            if (wave_active)
                                p.dbias_rows[(((size_t)bp.wh * (N / 16) + q0 / 16) * g.win + jy) * 64 + lane] = dacc;
                            dacc = 0.0f;
                        }
                    }
#pragma unroll
                    for (int c = 0; c < CT; ++c)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            dq[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                dS[r], Kt[(s * 16 + 4 * grp + r) * STR + 16 * c + r16], dq[c], 0, 0, 0);
                }
            }
        }
        if (it == ntiles - 1) {
            // end of pass 1: the 4 lane groups hold the same query, full row sum D_i
            Dq += __shfl_xor(Dq, 16);
            Dq += __shfl_xor(Dq, 32);
            if (wave_active && grp == 0) p.Dws[(size_t)bp.wh * N + qi] = Dq;
        }
        if (it + 1 < 2 * ntiles) store_tiles((it + 1) & 1, kst, vst);
        __syncthreads();
    };
    for (int it = 0; it < 2 * ntiles; it += 2) {   // 2 ntiles is even
        step(it, kreg, vreg, kreg2, vreg2);
        step(it + 1, kreg2, vreg2, kreg, vreg);
    }
    if (!wave_active) return;
    // lane holds dQ[query q0 + 4 grp + r][dim 16 c + r16]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float* orow = p.dQ + plane + (size_t)slot_pixel(g, bp.wy, bp.wx, q0 + 4 * grp + r) * D;
#pragma unroll
        for (int c = 0; c < CT; ++c) orow[16 * c + r16] = dq[c][r] * p.scale;
    }
}

template <typename T, int D, bool BIAS, bool HAS_DA>
__global__ __launch_bounds__(kBwdWaves * kWave, 4) void dense_bwd_dkv_kernel(const DenseBwdArgs p) {
    constexpr int DPL = D / 4;
    constexpr int CT = D / 16;
    constexpr int STR = D + 4;
    constexpr int SUB = kTile / 16;
    // SPLIT (d = 32, no bias): scores and dO.v on bf16 MFMA, the A operands (Q and dO
    // rows) from bf16 planes of the tiles made once per tile (double-buffered), the
    // fp32 Q/dO tiles that dV and dK multiply single-buffered (LDS for two
    // workgroups per CU)
    constexpr bool SPLIT = D == 32 && !BIAS;
    constexpr bool BFIN = sizeof(T) == 2;
    constexpr bool HOIST_DA = HAS_DA && !BIAS;
    constexpr int NB32 = SPLIT ? 1 : 2;
    constexpr int QPB = SPLIT ? (BFIN ? 1 : 3) * kTile * 64 : 16;
    constexpr int OPB = SPLIT ? 3 * kTile * 64 : 16;
    __shared__ __align__(16) float Qt2[NB32][kTile * STR];
    __shared__ __align__(16) float dOt2[NB32][kTile * STR];
    __shared__ __align__(16) unsigned char QP2[SPLIT ? 2 : 1][QPB];
    __shared__ __align__(16) unsigned char OP2[SPLIT ? 2 : 1][OPB];
    __shared__ float lset2[2][kTile];
    __shared__ float Dt2[2][kTile];
    __shared__ float btab[BIAS ? 63 * 63 : 1];

    const Geom g = p.g;
    const int N = g.N;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    const BlockPos bp = decode(g, (N + 16 * kBwdWaves - 1) / (16 * kBwdWaves), p.xcd_map);
    const int k0 = bp.blk * 16 * kBwdWaves + wave * 16;
    const bool wave_active = k0 < N;
    const size_t plane = (size_t)bp.bh * g.H * g.W * D;
    const T* Qh = static_cast<const T*>(p.Q) + plane;
    const T* Kh = static_cast<const T*>(p.K) + plane;
    const T* Vh = static_cast<const T*>(p.V) + plane;
    const float* dOh = p.dO + plane;
    const float sc = p.scale2;

    const int kj = wave_active ? k0 + r16 : 0;   // this lane's key (operand layout)
    float kv[DPL], vv[DPL];
    row_dims<T, D>(Kh + (size_t)slot_pixel(g, bp.wy, bp.wx, kj) * D, grp, kv);
    row_dims<T, D>(Vh + (size_t)slot_pixel(g, bp.wy, bp.wx, kj) * D, grp, vv);
    bf8 kh, km, kl, vh, vm, vl;   // SPLIT: this lane's 8 dims of k and v in parts
    if constexpr (SPLIT) {
        split3<8>(kv, kh, km, kl);
        split3<8>(vv, vh, vm, vl);
    }
    const int wrow = 2 * g.win - 1;
    int kbase = 0;   // bias index of (query at window row/col (0, 0), this key)
    if constexpr (BIAS) {
        const int nrel = wrow * wrow;
        const float* src = p.bias + (size_t)(bp.bh % g.heads) * nrel;
        for (int u = threadIdx.x; u < nrel; u += blockDim.x) btab[u] = src[u] * kLog2e;
        const int ky = kj / g.win;
        kbase = (g.win - 1 - ky) * wrow + g.win - 1 - (kj - ky * g.win);
    }
    const float* dAcol = HAS_DA ? p.dA + (size_t)bp.wh * N * N + kj : nullptr;

    v4f dv[CT], dk[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        dv[c] = v4f{0.f, 0.f, 0.f, 0.f};
        dk[c] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    // query tiles double-buffered: tile t + 1 (Q, dO, lse, D) is loaded into
    // registers while tile t is used from LDS
    const int ntiles = N / kTile;
    TileRegs<T, D> qreg;
    TileRegs<float, D> oreg;
    float lreg = 0.0f, dreg = 0.0f;
    auto load_small = [&](int t0) {
        if (threadIdx.x < kTile) {
            lreg = p.lse[(size_t)bp.wh * N + t0 + threadIdx.x] * kLog2e;
            dreg = p.Dws[(size_t)bp.wh * N + t0 + threadIdx.x];
        }
    };
    // SPLIT: planes, lse and D go to buffer b; the fp32 tiles to their single buffer
    auto store_buffered = [&](int b) {
        if constexpr (SPLIT) {
            qreg.store_planes64(QP2[b]);
            oreg.store_planes64(OP2[b]);
        } else {
            qreg.template store<STR>(Qt2[b]);
            oreg.template store<STR>(dOt2[b]);
        }
        if (threadIdx.x < kTile) {
            lset2[b][threadIdx.x] = lreg;
            Dt2[b][threadIdx.x] = dreg;
        }
    };
    auto store_fp32 = [&]() {
        qreg.template store<STR>(Qt2[0]);
        oreg.template store<STR>(dOt2[0]);
    };
    qreg.load(Qh, g, bp.wy, bp.wx, 0);
    oreg.load(dOh, g, bp.wy, bp.wx, 0);
    load_small(0);
    store_buffered(0);
    if constexpr (SPLIT) store_fp32();
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const int t0 = it * kTile;
        const float* Qt = Qt2[SPLIT ? 0 : (it & 1)];
        const float* dOt = dOt2[SPLIT ? 0 : (it & 1)];
        const float* lset = lset2[it & 1];
        const float* Dt = Dt2[it & 1];
        // this tile's dA^1 column values before the next tile's loads (waits count loads
        // in issue order), moved down by one 16-query step per step; with a bias table
        // they stay in the step (held here they spill)
        float dac[4 * SUB];
#pragma unroll
        for (int e = 0; e < 4 * SUB; ++e)
            dac[e] = HOIST_DA ? dAcol[(size_t)(t0 + (e >> 2) * 16 + 4 * grp + (e & 3)) * N] : 0.0f;
        if (it + 1 < ntiles) {
            qreg.load(Qh, g, bp.wy, bp.wx, t0 + kTile);
            oreg.load(dOh, g, bp.wy, bp.wx, t0 + kTile);
            load_small(t0 + kTile);
        }
        // not unrolled: the split operands of an unrolled loop spill under 128 VGPRs
        // (measured slower unrolled by 2 or 4)
#pragma unroll 1
        for (int s = 0; s < SUB; ++s) {
            const int qs = t0 + s * 16;   // queries qs + 4 grp + r of this lane
            v4f st = {0.f, 0.f, 0.f, 0.f}, dpt = {0.f, 0.f, 0.f, 0.f};
            if constexpr (SPLIT) {
                // A rows: queries s*16 + r16, dims 8 grp .. 8 grp + 7 (swizzled chunk)
                const int row = s * 16 + r16;
                const int off = row * 64 + ((grp ^ ((row >> 2) & 3)) << 4);
                const unsigned char* qp = QP2[it & 1] + off;
                const unsigned char* op = OP2[it & 1] + off;
                const bf8 qh = *reinterpret_cast<const bf8*>(qp);
                const bf8 dh = *reinterpret_cast<const bf8*>(op);
                const bf8 dm = *reinterpret_cast<const bf8*>(op + kTile * 64);
                const bf8 dl = *reinterpret_cast<const bf8*>(op + 2 * kTile * 64);
                if constexpr (BFIN) {   // q, k, v exact in bf16: one product; dO in three parts
                    st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, kh, st, 0, 0, 0);
                    dpt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dl, vh, dpt, 0, 0, 0);
                    dpt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dm, vh, dpt, 0, 0, 0);
                    dpt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dh, vh, dpt, 0, 0, 0);
                } else {
                    const bf8 qm = *reinterpret_cast<const bf8*>(qp + kTile * 64);
                    const bf8 ql = *reinterpret_cast<const bf8*>(qp + 2 * kTile * 64);
                    st = dot_split3(qh, qm, ql, kh, km, kl, st);
                    dpt = dot_split3(dh, dm, dl, vh, vm, vl, dpt);
                }
            } else {
                const float* qr = Qt + (s * 16 + r16) * STR + DPL * grp;
                const float* dr = dOt + (s * 16 + r16) * STR + DPL * grp;
#pragma unroll
                for (int x = 0; x < DPL; ++x) {
                    st = __builtin_amdgcn_mfma_f32_16x16x4f32(qr[x], kv[x], st, 0, 0, 0);
                    dpt = __builtin_amdgcn_mfma_f32_16x16x4f32(dr[x], vv[x], dpt, 0, 0, 0);
                }
            }
            float b[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (BIAS) {
                const int qa = qs + 4 * grp;
                const int qy = qa / g.win;
                const int idx0 = kbase + qy * wrow + (qa - qy * g.win);
#pragma unroll
                for (int r = 0; r < 4; ++r) b[r] = btab[idx0 + r];
            }
            float P[4], dS[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ql = s * 16 + 4 * grp + r;   // query within the tile
                P[r] = fast_exp2(fmaf(st[r], sc, b[r] - lset[ql]));
                const float G = dpt[r] + (HOIST_DA ? dac[r] : HAS_DA ? dAcol[(size_t)(t0 + ql) * N] : 0.0f);
                dS[r] = P[r] * (G - Dt[ql]);
            }
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int ql = s * 16 + 4 * grp + r;
                    dv[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(P[r], dOt[ql * STR + 16 * c + r16], dv[c], 0, 0, 0);
                    dk[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(dS[r], Qt[ql * STR + 16 * c + r16], dk[c], 0, 0, 0);
                }
#pragma unroll
            for (int e = 0; e < 4 * (SUB - 1); ++e) dac[e] = dac[e + 4];
        }
        if (it + 1 < ntiles) store_buffered((it + 1) & 1);
        if constexpr (SPLIT) {
            // every wave is done with the fp32 tile before the next one replaces it
            __syncthreads();
            if (it + 1 < ntiles) store_fp32();
        }
        __syncthreads();
    }
    if (!wave_active) return;
    // lane holds dV / dK[key k0 + 4 grp + r][dim 16 c + r16]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const size_t o = plane + (size_t)slot_pixel(g, bp.wy, bp.wx, k0 + 4 * grp + r) * D;
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            p.dV[o + 16 * c + r16] = dv[c][r];
            p.dK[o + 16 * c + r16] = dk[c][r] * p.scale;
        }
    }
}

template <typename T, int D, bool BIAS, bool HAS_DA>
hipError_t launch_dbwd_t(const DenseBwdArgs& a, int grid, hipStream_t s) {
    if constexpr (BIAS) {
        if (a.dbias_rows)
            hipLaunchKernelGGL((dense_bwd_dq_kernel<T, D, true, HAS_DA, true>), dim3(grid), dim3(kBwdWaves * kWave),
                               0, s, a);
        else
            hipLaunchKernelGGL((dense_bwd_dq_kernel<T, D, true, HAS_DA, false>), dim3(grid), dim3(kBwdWaves * kWave),
                               0, s, a);
    } else {
        hipLaunchKernelGGL((dense_bwd_dq_kernel<T, D, false, HAS_DA, false>), dim3(grid), dim3(kBwdWaves * kWave), 0,
                           s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dense_bwd_dkv_kernel<T, D, BIAS, HAS_DA>), dim3(grid), dim3(kBwdWaves * kWave), 0, s, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dbwd_d(const DenseBwdArgs& a, int grid, hipStream_t s) {
    if (a.bias) return a.dA ? launch_dbwd_t<T, D, true, true>(a, grid, s) : launch_dbwd_t<T, D, true, false>(a, grid, s);
    return a.dA ? launch_dbwd_t<T, D, false, true>(a, grid, s) : launch_dbwd_t<T, D, false, false>(a, grid, s);
}

}  // namespace

int dense_bwd_blocks(int N) { return (N + 16 * kBwdWaves - 1) / (16 * kBwdWaves); }

hipError_t launch_dense_backward(const DenseBwdArgs& a, int dtype, int D, int grid, hipStream_t stream) {
    if (dtype == 0)
        return D == 16 ? launch_dbwd_d<float, 16>(a, grid, stream) : launch_dbwd_d<float, 32>(a, grid, stream);
    return D == 16 ? launch_dbwd_d<uint16_t, 16>(a, grid, stream) : launch_dbwd_d<uint16_t, 32>(a, grid, stream);
}

}  // namespace pfa
