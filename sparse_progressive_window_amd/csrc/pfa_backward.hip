// Backward pass of a window-mode sparse PFA layer on gfx950, kept sets fixed.
//
// Forward, per query slot i with kept slots r = 1..K_l (paper notes "Progressive
// Focused Transformer for Single Image Super-Resolution", sections "Progressive
// attention across layers" and "Sparse matrix multiplication"):
//   A_ir = A^{l-1}_ir exp(s_ir) / sum_kept A^{l-1} exp(s),  s_ir = q_i.k_j / sqrt(d),
//   O_i  = sum_r A_ir v_j.
// Both normalisations and the softmax denominator over the candidate list are
// row constants, so A^l is a softmax over the kept slots of the log-domain key
// s + ln A^{l-1}. With G_ir = dA_ir + dO_i.v_j and g_ir = G_ir - sum_r A_ir G_ir:
//   dkey_ir     = A_ir g_ir                     (softmax backward)
//   dQ_i        = sum_r dkey_ir k_j / sqrt(d)
//   dK_j       += dkey_ir q_i / sqrt(d)
//   dV_j       += A_ir dO_i
//   dA^{l-1}_ir = dkey_ir / A^{l-1}_ir  at kept slots, 0 at dropped ones.
//
// Kernels.
// * bwd_rows_kernel: one group of GL lanes per query row; CH lanes split each
//   16-byte chunked V/K row (CH = row bytes / 16) and a subgroup of CH lanes
//   takes 4 consecutive kept slots at a time. Pass V: gather v_j from LDS, dot
//   with dO_i (chunk sums by DPP quad exchanges and a half-row mirror), row sum
//   D_i, g written to a workspace; alone with 8 chunk lanes (fp32, d = 32) a
//   transposing reduction leaves one entry per lane, so a lane loads only that
//   entry's A and dA, and the next row's loads go out before this row's
//   reduction and stores. Pass K: gather k_j from LDS, dQ_i, and
//   dA^{l-1}: kept tokens are marked in a per-row LDS bitmap, the I^{l-1} row is
//   scanned in slot order, and the r-th marked slot takes kept entry r (I^l is
//   a subsequence of I^{l-1} in its order). When K and V fit in LDS together
//   both passes run in one kernel, keeping G in registers.
// * bwd_dkv_kernel (N a multiple of 16): dV = A^T dO and dK = (A g)^T Q / sqrt(d)
//   as dense fp32 MFMA products over row blocks densified in LDS, the dV / dK
//   tiles of each wave's tokens held in registers. At the densities of the keep
//   schedule (K_l / N from 1/4 down to 1/64) this beats accumulating through
//   LDS: on gfx950 an LDS fp32 atomic add retires at ~190 clocks per wavefront
//   instruction and a compare-and-swap loop still costs tens.
// * bwd_scatter_kernel (other N): dK and dV accumulate in LDS (fp32, DH of the
//   d columns per workgroup) by compare-and-swap adds; each wave stages one
//   row's (j, A, A g/sqrt(d)) in LDS and its lanes cover (64/DH kept slots) x
//   DH columns per instruction.
#include "pfa_kernels.h"
#include "pfa_rows.h"

namespace pfa {
namespace {

constexpr int kBwdRowWaves = 16;
constexpr int kBwdScatterWaves = 8;

// sum over the CH consecutive lanes that share a kept slot (CH = 2, 4 or 8)
template <int CH>
__device__ __forceinline__ float chunk_sum(float v) {
    if (CH >= 2) v += dppf<kQuadXor1>(v);
    if (CH >= 4) v += dppf<kQuadXor2>(v);
    if (CH >= 8) v += dppf<kRowHalfMirror>(v);
    return v;
}

// sum over the lanes of a GL-lane group that hold the same chunk (lane bits
// [log2 CH, log2 GL)); once per row, so plain cross-lane shuffles
template <int CH, int GL>
__device__ __forceinline__ float subgroup_sum(float v) {
#pragma unroll
    for (int o = CH; o < GL; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

// bits of the wave mask m that belong to this lane's GL-lane group, and the
// number of them below this lane
template <int GL>
__device__ __forceinline__ uint64_t group_bits(uint64_t m, int lane) {
    if (GL == 64) return m;
    return (m >> (lane & (64 - GL))) & ((1ull << GL) - 1ull);
}

// Two fp32 adds into LDS words by compare-and-swap (ds_cmpst_rtn_b32): on gfx950
// LDS fp32 atomic adds (ds_add_f32) retire at ~190 clocks per wavefront
// instruction, 32-bit integer atomics at ~4.5. The lanes of one instruction
// target distinct words, so a retry only follows an update by another wave.
__device__ __forceinline__ void lds_add2(unsigned* a, float va, unsigned* b, float vb) {
    unsigned oa = *a, ob = *b;
    bool da = false, db = false;
    do {
        if (!da) {
            unsigned e = oa;
            da = __hip_atomic_compare_exchange_strong(a, &e, __float_as_uint(__uint_as_float(oa) + va),
                                                      __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            oa = e;
        }
        if (!db) {
            unsigned e = ob;
            db = __hip_atomic_compare_exchange_strong(b, &e, __float_as_uint(__uint_as_float(ob) + vb),
                                                      __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            ob = e;
        }
    } while (!(da && db));
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <typename T, int D>
__device__ __forceinline__ void load_row_chunk(const T* row, int chunk, float (&o)[Chunk<T>::kElems]) {
    Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(reinterpret_cast<const unsigned char*>(row) + chunk * 16), o);
}

template <typename T, int D, int GL, int NST, bool HAS_V, bool HAS_K>
__global__ __launch_bounds__(kBwdRowWaves * kWave) void bwd_rows_kernel(const BackwardArgs p) {
    constexpr int NW = kBwdRowWaves;
    constexpr int EPC = Chunk<T>::kElems;   // elements per 16-byte chunk
    constexpr int CH = D / EPC;             // chunks (lanes) per K/V row
    constexpr int ROWB = D * (int)sizeof(T);
    constexpr int GS = GL / CH;             // subgroups per row group
    constexpr int RPW = kWave / GL;         // rows per wavefront
    constexpr int KPL = 4 * NST;            // kept slots per lane
    static_assert(CH >= 2 && CH <= 8 && GS >= 1, "row split");
    extern __shared__ __align__(16) unsigned char smem[];

    const Geom g = p.g;
    const int N = g.N;
    const int K_l = p.K_l;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int grp = lane / GL;
    const int gl = lane & (GL - 1);
    const int vchunk = gl % CH;
    const int vsub = gl / CH;
    const WhPart w = decode_block(p.blocks_per_wh, p.xcd_map, g);
    const size_t plane = (size_t)w.bh * g.H * g.W * D;

    unsigned char* Vs = smem;
    unsigned char* Ks = smem + (HAS_V ? N * ROWB : 0);
    const bool want_dap = HAS_K && p.dA_prev != nullptr;
    const int bmw = (N + 31) >> 5;                       // bitmap words per row
    const int rsw = bmw + ((K_l + 3) & ~3);              // row scratch words
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(smem + (HAS_V + HAS_K) * N * ROWB) + (wave * RPW + grp) * rsw;
    float* vals = reinterpret_cast<float*>(bitmap + bmw);
    if (HAS_V) stage_rows<T, D>(Vs, ROWB, static_cast<const T*>(p.V) + plane, g, w.wy, w.wx);
    if (HAS_K) stage_rows<T, D>(Ks, ROWB, static_cast<const T*>(p.K) + plane, g, w.wy, w.wx);
    __syncthreads();

    const size_t wh_pairs = (size_t)w.wh * N * K_l;
    const int pair_bytes = N * K_l * 4;
    const __amdgpu_buffer_rsrc_t rI = make_rsrc(p.I_l + wh_pairs, pair_bytes);
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A_l + wh_pairs, pair_bytes);
    const __amdgpu_buffer_rsrc_t rdA = make_rsrc(p.dA_l ? p.dA_l + wh_pairs : p.A_l, p.dA_l ? pair_bytes : 0);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.g_buf + wh_pairs, pair_bytes);
    const int row0 = w.part * p.rows_per_block;
    const int row1 = min(N, row0 + p.rows_per_block);

    if constexpr (HAS_V && !HAS_K && CH == 8) {
        // V pass alone with 8 chunk lanes per row (fp32, d = 32). The 4 entries of a
        // step are summed over their chunk lanes by a transposing reduction (each
        // stage sends half of the partial sums), which leaves lane c with entry ent
        // of the step; lanes c and 7 - c agree. A lane therefore loads the step's 4
        // slot indices (all chunk lanes gather their V chunks) but only its own
        // entry's A and dA, and a row's loads are issued while the previous row is
        // reduced and its g stored.
        const int hh = (vchunk >> 2) & 1;
        const int b0 = (vchunk & 1) ^ hh;
        const int b1 = ((vchunk >> 1) & 1) ^ hh;
        const int ent = 2 * b0 + b1;
        struct VRow {
            uint4 j4[NST];
            float av[NST], dv[NST];
            float4 dO;
        };
        auto load_vrow = [&](VRow& r, int ii) {
            const int roff = ii * K_l * 4;
            r.dO = *reinterpret_cast<const float4*>(p.dO + plane + (size_t)slot_pixel(g, w.wy, w.wx, ii) * D +
                                                    vchunk * EPC);
#pragma unroll
            for (int t = 0; t < NST; ++t) {
                const int off = roff + 4 * (vsub + GS * t) * 4;
                r.j4[t] = load16(rI, off);
                r.av[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rA, off + ent * 4, 0, 0));
                r.dv[t] = p.dA_l ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdA, off + ent * 4, 0, 0))
                                 : 0.0f;
            }
        };
        int base = row0 + wave * RPW;
        VRow cur;
        if (base < row1) load_vrow(cur, base + grp < row1 ? base + grp : row0);
        for (; base < row1; base += NW * RPW) {
            const int i = base + grp;
            const bool active = i < row1;
            const int roff = (active ? i : row0) * K_l * 4;
            VRow nxt;
            const int nb = base + NW * RPW;
            if (nb < row1) load_vrow(nxt, nb + grp < row1 ? nb + grp : row0);
            const float dov[4] = {cur.dO.x, cur.dO.y, cur.dO.z, cur.dO.w};
            float Gt[NST];
            float dsum = 0.0f;
#pragma unroll
            for (int t = 0; t < NST; ++t) {
                const int e0 = 4 * (vsub + GS * t);
                const unsigned jv[4] = {cur.j4[t].x, cur.j4[t].y, cur.j4[t].z, cur.j4[t].w};
                float part[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int j = (int)min(jv[x], (unsigned)(N - 1));   // memory safety only
                    float vf[EPC];
                    Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(Vs + j * ROWB + vchunk * 16), vf);
                    float sdot = 0.0f;
#pragma unroll
                    for (int y = 0; y < EPC; ++y) sdot = fmaf(dov[y], vf[y], sdot);
                    part[x] = sdot;
                }
                // keep entries 2 b0, 2 b0 + 1; the other two go to lane c ^ 1
                const float r0 = (b0 ? part[2] : part[0]) + dppf<kQuadXor1>(b0 ? part[0] : part[2]);
                const float r1 = (b0 ? part[3] : part[1]) + dppf<kQuadXor1>(b0 ? part[1] : part[3]);
                // keep entry 2 b0 + b1; the other goes to lane c ^ 2
                const float r2 = (b1 ? r1 : r0) + dppf<kQuadXor2>(b1 ? r0 : r1);
                // lane 7 - c holds the same entry
                const float tot = r2 + dppf<kRowHalfMirror>(r2);
                const bool valid = e0 + ent < K_l;
                const float gx = valid ? cur.dv[t] + tot : 0.0f;
                Gt[t] = gx;
                dsum = fmaf((valid && hh == 0) ? cur.av[t] : 0.0f, gx, dsum);   // one lane per entry
            }
            dsum = chunk_sum<CH>(dsum);   // the 4 entries of each lane quad
            const float Dsum = subgroup_sum<CH, GL>(dsum);
#pragma unroll
            for (int t = 0; t < NST; ++t) {
                const int e0 = 4 * (vsub + GS * t);
                const bool st = active && hh == 0 && e0 + ent < K_l;   // the lower 4 lanes store
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Gt[t] - Dsum), rg,
                                                      st ? roff + (e0 + ent) * 4 : 0x7FFFFFF0, 0, 0);
            }
            cur = nxt;
        }
        return;
    }

    // K pass alone: a row's query chunk and first-step loads are issued before the
    // previous row's dA^{l-1} scan, whose stores would otherwise delay them (one
    // in-order wait counter for loads and stores)
    constexpr bool XR = HAS_K && !HAS_V;
    float qvx[EPC];
    uint4 j4x = make_uint4(0u, 0u, 0u, 0u), a4x = j4x, g4x = j4x;
    auto load_first = [&](int b0) {
        const int ix = b0 + grp < row1 ? b0 + grp : row0;
        load_row_chunk<T, D>(static_cast<const T*>(p.Q) + plane + (size_t)slot_pixel(g, w.wy, w.wx, ix) * D, vchunk,
                             qvx);
        const int ro = ix * K_l * 4 + 16 * vsub;
        j4x = load16(rI, ro);
        a4x = load16(rA, ro);
        g4x = load16(rg, ro);
    };
    if constexpr (XR) {
        if (row0 + wave * RPW < row1) load_first(row0 + wave * RPW);
    }
    // K and V pass: the next row's dO chunk and first-step loads, likewise
    constexpr bool XV = HAS_K && HAS_V && NST <= 2;   // with more steps the carried loads spill
    float dovx[EPC];
    uint4 j4v = make_uint4(0u, 0u, 0u, 0u), a4v = j4v, d4v = j4v;
    auto load_first_v = [&](int b0) {
        const int ix = b0 + grp < row1 ? b0 + grp : row0;
        const float* dor = p.dO + plane + (size_t)slot_pixel(g, w.wy, w.wx, ix) * D + vchunk * EPC;
#pragma unroll
        for (int y = 0; y < EPC; y += 4) {
            const float4 f = *reinterpret_cast<const float4*>(dor + y);
            dovx[y] = f.x; dovx[y + 1] = f.y; dovx[y + 2] = f.z; dovx[y + 3] = f.w;
        }
        const int ro = ix * K_l * 4 + 16 * vsub;
        j4v = load16(rI, ro);
        a4v = load16(rA, ro);
        d4v = p.dA_l ? load16(rdA, ro) : make_uint4(0u, 0u, 0u, 0u);
    };
    if constexpr (XV) {
        if (row0 + wave * RPW < row1) load_first_v(row0 + wave * RPW);
    }
    for (int base = row0 + wave * RPW; base < row1; base += NW * RPW) {
        const int i = base + grp;
        const bool active = i < row1;
        const int ii = active ? i : row0;          // idle groups work on a valid row and store nothing
        const int qpix = slot_pixel(g, w.wy, w.wx, ii);
        const int roff = ii * K_l * 4;             // byte offset of the row's kept slots

        float G[HAS_V ? KPL : 1];
        if (HAS_V) {
            float dov[EPC];
            if constexpr (XV) {
#pragma unroll
                for (int y = 0; y < EPC; ++y) dov[y] = dovx[y];
            } else {
                const float* dor = p.dO + plane + (size_t)qpix * D + vchunk * EPC;
#pragma unroll
                for (int y = 0; y < EPC; y += 4) {
                    const float4 f = *reinterpret_cast<const float4*>(dor + y);
                    dov[y] = f.x; dov[y + 1] = f.y; dov[y + 2] = f.z; dov[y + 3] = f.w;
                }
            }
            float dsum = 0.0f;
#pragma unroll
            for (int t = 0; t < NST; ++t) {
                const int e0 = 4 * (vsub + GS * t);
                const int off = roff + e0 * 4;
                const uint4 j4 = (XV && t == 0) ? j4v : load16(rI, off);
                const uint4 a4 = (XV && t == 0) ? a4v : load16(rA, off);
                const uint4 d4 = (XV && t == 0) ? d4v : p.dA_l ? load16(rdA, off) : make_uint4(0u, 0u, 0u, 0u);
                const unsigned jv[4] = {j4.x, j4.y, j4.z, j4.w};
                const float av[4] = {__uint_as_float(a4.x), __uint_as_float(a4.y), __uint_as_float(a4.z),
                                     __uint_as_float(a4.w)};
                const float dv[4] = {__uint_as_float(d4.x), __uint_as_float(d4.y), __uint_as_float(d4.z),
                                     __uint_as_float(d4.w)};
                float part[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int j = (int)min(jv[x], (unsigned)(N - 1));   // memory safety only
                    float vf[EPC];
                    Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(Vs + j * ROWB + vchunk * 16), vf);
                    float s = 0.0f;
#pragma unroll
                    for (int y = 0; y < EPC; ++y) s = fmaf(dov[y], vf[y], s);
                    part[x] = s;
                }
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const bool valid = e0 + x < K_l;
                    const float gx = valid ? dv[x] + chunk_sum<CH>(part[x]) : 0.0f;
                    G[4 * t + x] = gx;
                    dsum = fmaf(valid ? av[x] : 0.0f, gx, dsum);
                }
            }
            const float Dsum = subgroup_sum<CH, GL>(dsum);
#pragma unroll
            for (int k = 0; k < KPL; ++k) G[k] -= Dsum;
            // g for the scatter pass (and the K pass): lane x % CH of a subgroup stores slot x
#pragma unroll
            for (int t = 0; t < NST; ++t) {
                const int e0 = 4 * (vsub + GS * t);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    if (x % CH != vchunk) continue;
                    const bool st = active && e0 + x < K_l;
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(G[4 * t + x]), rg,
                                                          st ? roff + (e0 + x) * 4 : 0x7FFFFFF0, 0, 0);
                }
            }
        }

        if (HAS_K) {
            float qv[EPC];
            if constexpr (XR) {
#pragma unroll
                for (int y = 0; y < EPC; ++y) qv[y] = qvx[y];
            } else {
                load_row_chunk<T, D>(static_cast<const T*>(p.Q) + plane + (size_t)qpix * D, vchunk, qv);
            }
            float dq[EPC];
#pragma unroll
            for (int y = 0; y < EPC; ++y) dq[y] = 0.0f;
            if (want_dap) {
                for (int u = gl; u < bmw; u += GL) bitmap[u] = 0u;
            }
            // without V in this kernel g comes from the workspace, one step at a time:
            // the next step's loads are issued before this step's gathers, and the
            // loop is unrolled by 2 (measured 7-8 % faster than rolled; by 4 or fully
            // the hoisted loads spill)
            constexpr int KUN = HAS_V ? NST : 2;   // steps unrolled
            uint4 j4n = XR ? j4x : load16(rI, roff + 16 * vsub);
            uint4 a4n = XR ? a4x : load16(rA, roff + 16 * vsub);
            uint4 g4n = HAS_V ? make_uint4(0u, 0u, 0u, 0u) : XR ? g4x : load16(rg, roff + 16 * vsub);
#pragma unroll KUN
            for (int t = 0; t < NST; ++t) {
                const int e0 = 4 * (vsub + GS * t);
                const uint4 j4 = j4n;
                const uint4 a4 = a4n;
                const uint4 g4 = g4n;
                if (t + 1 < NST) {
                    const int offn = roff + (e0 + 4 * GS) * 4;
                    j4n = load16(rI, offn);
                    a4n = load16(rA, offn);
                    if (!HAS_V) g4n = load16(rg, offn);
                }
                float gv[4];
                if (HAS_V) {
#pragma unroll
                    for (int x = 0; x < 4; ++x) gv[x] = G[4 * t + x];
                } else {
                    gv[0] = __uint_as_float(g4.x);
                    gv[1] = __uint_as_float(g4.y);
                    gv[2] = __uint_as_float(g4.z);
                    gv[3] = __uint_as_float(g4.w);
                }
                const unsigned jv[4] = {j4.x, j4.y, j4.z, j4.w};
                const float av[4] = {__uint_as_float(a4.x), __uint_as_float(a4.y), __uint_as_float(a4.z),
                                     __uint_as_float(a4.w)};
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const bool valid = e0 + x < K_l;
                    const int j = (int)min(jv[x], (unsigned)(N - 1));
                    const float dkey = valid ? av[x] * gv[x] : 0.0f;
                    float kf[EPC];
                    Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(Ks + j * ROWB + vchunk * 16), kf);
#pragma unroll
                    for (int y = 0; y < EPC; ++y) dq[y] = fmaf(dkey, kf[y], dq[y]);
                    if (want_dap && valid && x % CH == vchunk) {
                        vals[e0 + x] = dkey;
                        atomicOr(&bitmap[j >> 5], 1u << (j & 31));
                    }
                }
            }
#pragma unroll
            for (int y = 0; y < EPC; ++y) dq[y] = subgroup_sum<CH, GL>(dq[y]) * p.scale;
            if (active && vsub == 0) {
                float* qr = p.dQ + plane + (size_t)qpix * D + vchunk * EPC;
#pragma unroll
                for (int y = 0; y < EPC; y += 4)
                    *reinterpret_cast<float4*>(qr + y) = make_float4(dq[y], dq[y + 1], dq[y + 2], dq[y + 3]);
            }
            if constexpr (XR) {
                if (base + NW * RPW < row1) load_first(base + NW * RPW);
            }
            if constexpr (XV) {
                if (base + NW * RPW < row1) load_first_v(base + NW * RPW);
            }
            if (want_dap) {
                // the wave's LDS writes above complete before the scan reads them
                __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                // the row's slots in chunks of SU x GL, each chunk's loads issued together and
                // before the previous chunk's stores: stores count in the same in-order
                // vector-memory counter, so loads issued after them would wait for them too
                // (measured 17 % faster on the 1024-slot rows; 8 x GL slots beats 4 and 16)
                constexpr int SU = NST >= 8 ? 8 : 4;
                const int K_prev = p.K_prev;
                const size_t srow = ((size_t)w.wh * N + ii) * K_prev;
                int run = 0;
                int jn[SU];
                float an[SU];
                auto load_chunk = [&](int s0) {
#pragma unroll
                    for (int u = 0; u < SU; ++u) {
                        const int slot = s0 + u * GL + gl;
                        jn[u] = slot;
                        an[u] = 0.0f;
                        if (slot < K_prev) {
                            if (p.I_prev) jn[u] = p.I_prev[srow + slot];
                            an[u] = p.A_prev[srow + slot];
                        }
                    }
                };
                load_chunk(0);
                for (int s0 = 0; s0 < K_prev; s0 += SU * GL) {
                    int jj[SU];
                    float ap[SU];
#pragma unroll
                    for (int u = 0; u < SU; ++u) { jj[u] = jn[u]; ap[u] = an[u]; }
                    if (s0 + SU * GL < K_prev) load_chunk(s0 + SU * GL);
#pragma unroll
                    for (int u = 0; u < SU; ++u) {
                        const int slot = s0 + u * GL + gl;
                        const bool sv = slot < K_prev;
                        const int j = (int)min((unsigned)jj[u], (unsigned)(N - 1));
                        const bool kept = sv && ((bitmap[j >> 5] >> (j & 31)) & 1u);
                        const uint64_t m = group_bits<GL>(ballot(kept), lane);
                        const int rank = run + __builtin_popcountll(m & ((1ull << gl) - 1ull));
                        run += __builtin_popcountll(m);
                        // v_rcp_f32 (1 ulp) and a product instead of the IEEE division
                        // sequence (~10 instructions per slot, every slot of the row)
                        float val = 0.0f;
                        if (kept && rank < K_l && ap[u] > 0.0f) val = vals[rank] * __builtin_amdgcn_rcpf(ap[u]);
                        if (active && sv) p.dA_prev[srow + slot] = val;
                    }
                }
            }
        }
    }
}

template <typename T, int D, int DH>
__global__ __launch_bounds__(kBwdScatterWaves * kWave) void bwd_scatter_kernel(const BackwardArgs p) {
    constexpr int NW = kBwdScatterWaves;
    constexpr int PPI = kWave / DH;         // kept slots per atomic instruction
    extern __shared__ __align__(16) unsigned char smem[];

    const Geom g = p.g;
    const int N = g.N;
    const int K_l = p.K_l;
    const int KLP = (K_l + 3) & ~3;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const WhPart w = decode_block(p.blocks_per_wh, p.xcd_map, g);   // part = column block
    const size_t plane = (size_t)w.bh * g.H * g.W * D;
    const int col0 = w.part * DH;

    float* accV = reinterpret_cast<float*>(smem);
    float* accK = accV + N * DH;
    int* st_j = reinterpret_cast<int*>(accK + N * DH) + wave * 3 * KLP;
    float* st_a = reinterpret_cast<float*>(st_j + KLP);
    float* st_k = st_a + KLP;
    for (int u = threadIdx.x * 4; u < 2 * N * DH; u += blockDim.x * 4)
        *reinterpret_cast<float4*>(accV + u) = make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();

    const size_t wh_pairs = (size_t)w.wh * N * K_l;
    const int pair_bytes = N * K_l * 4;
    const __amdgpu_buffer_rsrc_t rI = make_rsrc(p.I_l + wh_pairs, pair_bytes);
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A_l + wh_pairs, pair_bytes);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.g_buf + wh_pairs, pair_bytes);
    const int c = lane % DH;
    const int ps = lane / DH;
    const T* Qh = static_cast<const T*>(p.Q) + plane;
    for (int i = wave; i < N; i += NW) {
        const int qpix = slot_pixel(g, w.wy, w.wx, i);
        const float dov = p.dO[plane + (size_t)qpix * D + col0 + c];
        float qv;
        if constexpr (sizeof(T) == 4) {
            qv = reinterpret_cast<const float*>(Qh)[(size_t)qpix * D + col0 + c];
        } else {
            qv = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(Qh)[(size_t)qpix * D + col0 + c] << 16);
        }
        const int roff = i * K_l * 4;
        for (int e = lane * 4; e < K_l; e += 4 * kWave) {
            const uint4 j4 = load16(rI, roff + e * 4);
            const uint4 a4 = load16(rA, roff + e * 4);
            const uint4 g4 = load16(rg, roff + e * 4);
            const float a[4] = {__uint_as_float(a4.x), __uint_as_float(a4.y), __uint_as_float(a4.z),
                                __uint_as_float(a4.w)};
            const float gg[4] = {__uint_as_float(g4.x), __uint_as_float(g4.y), __uint_as_float(g4.z),
                                 __uint_as_float(g4.w)};
            *reinterpret_cast<uint4*>(st_j + e) = j4;
            *reinterpret_cast<float4*>(st_a + e) = make_float4(a[0], a[1], a[2], a[3]);
            *reinterpret_cast<float4*>(st_k + e) = make_float4(a[0] * gg[0] * p.scale, a[1] * gg[1] * p.scale,
                                                               a[2] * gg[2] * p.scale, a[3] * gg[3] * p.scale);
        }
        for (int e0 = 0; e0 < K_l; e0 += PPI) {
            const int e = e0 + ps;
            if (e < K_l) {
                const int j = (int)min((unsigned)st_j[e], (unsigned)(N - 1));
                lds_add2(reinterpret_cast<unsigned*>(accV + j * DH + c), st_a[e] * dov,
                         reinterpret_cast<unsigned*>(accK + j * DH + c), st_k[e] * qv);
            }
        }
    }
    __syncthreads();
    constexpr int C4 = DH / 4;
    for (int u = threadIdx.x; u < N * C4; u += blockDim.x) {
        const int t = u / C4;
        const int cc = (u - t * C4) * 4;
        const size_t o = plane + (size_t)slot_pixel(g, w.wy, w.wx, t) * D + col0 + cc;
        *reinterpret_cast<float4*>(p.dV + o) = *reinterpret_cast<const float4*>(accV + t * DH + cc);
        *reinterpret_cast<float4*>(p.dK + o) = *reinterpret_cast<const float4*>(accK + t * DH + cc);
    }
}

// dV = A^T dO and dK = (A g / sqrt(d))^T Q for one window-head on fp32 MFMA
// (v_mfma_f32_16x16x4_f32: exact products, fp32 accumulation). The kept rows are
// densified in LDS, KB = 16 rows at a time (two [KB][N] fp32 planes: A and
// A g / sqrt(d), zero off the kept slots), next to the block's dO and Q rows;
// wave w owns tokens [16 MTW w, 16 MTW (w + 1)) and keeps their dV and dK tiles in
// registers over all blocks, so nothing is accumulated through memory. The next
// block's (j, A, g) entries are loaded into registers during the current block's
// MFMAs; after the MFMAs the written slots are reset to zero.
template <typename T, int D, int EPT, int MTW, bool SKIP>
__global__ __launch_bounds__(16 * kWave) void bwd_dkv_kernel(const BackwardArgs p) {
    constexpr int KB = 16;                  // rows per block (4 MFMA k-steps)
    constexpr int NT = D / 16;              // 16-column tiles of d
    constexpr int XS = D == 32 ? 48 : 16;   // X row stride: 4 rows x 16 columns cover 64 distinct banks
    typedef float v4f __attribute__((ext_vector_type(4)));
    extern __shared__ __align__(16) unsigned char smem[];

    const Geom g = p.g;
    const int N = g.N;
    const int K_l = p.K_l;
    const int NP = N + 16;                  // dense row stride: 4 rows x 16 columns cover 64 distinct banks
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r16 = lane & 15;
    const int q4 = lane >> 4;
    // a whole window-head, or one token half of a window-head (see dkv_full)
    WhPart w;
    int half = -1;
    if ((int)blockIdx.x < p.dkv_full) {
        w = decode_block(1, p.xcd_map, g);
    } else {
        const int s = (int)blockIdx.x - p.dkv_full;
        w = wh_coords(p.dkv_full + (s >> 4) * 8 + (s & 7), 0, g);
        half = (s >> 3) & 1;
    }
    const size_t plane = (size_t)w.bh * g.H * g.W * D;
    const T* Qh = static_cast<const T*>(p.Q) + plane;
    const float* dOh = p.dO + plane;

    float* Md = reinterpret_cast<float*>(smem);      // [2][KB][NP]
    float* Xs = Md + 2 * KB * NP;                    // [2][KB][XS]: dO rows, Q rows
    for (int u = threadIdx.x * 4; u < 2 * KB * NP; u += blockDim.x * 4)
        *reinterpret_cast<float4*>(Md + u) = make_float4(0.f, 0.f, 0.f, 0.f);

    const size_t wh_pairs = (size_t)w.wh * N * K_l;
    const int pair_bytes = N * K_l * 4;
    const __amdgpu_buffer_rsrc_t rI = make_rsrc(p.I_l + wh_pairs, pair_bytes);
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A_l + wh_pairs, pair_bytes);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.g_buf + wh_pairs, pair_bytes);
    const int mtiles = N / 16;                       // a multiple of MTW, at most 16 MTW
    // this workgroup's token tiles [tile0, tile0 + btiles), mtw per wave (MTW even
    // when halves are launched)
    const int btiles = half < 0 ? mtiles : mtiles / 2;
    const int tile0 = half < 0 ? 0 : half * btiles;
    const int mtw = half < 0 ? MTW : MTW / 2;
    const bool wave_active = wave * mtw < btiles;
    const int nblk = N / KB;
    const int blk_entries = KB * K_l;

    // entries of block b: e = threadIdx.x + 1024 u, row b*KB + e / K_l, slot e % K_l
    // (the row inside the block is the same for every block)
    int erow[EPT];
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
        const int e = threadIdx.x + 1024 * u;
        erow[u] = e < blk_entries ? e / K_l : -1;
    }
    unsigned ej[EPT];
    float ea[EPT], ek[EPT];
    auto load_block = [&](int b) {
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = threadIdx.x + 1024 * u;
            const int off = erow[u] >= 0 ? (b * blk_entries + e) * 4 : 0x7FFFFFF0;   // dropped past the rows
            ej[u] = __builtin_amdgcn_raw_buffer_load_b32(rI, off, 0, 0);
            const float a = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rA, off, 0, 0));
            const float gg = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, off, 0, 0));
            ea[u] = a;
            ek[u] = a * gg * p.scale;
        }
    };
    // the block's dO and Q rows (fp32), one value per thread while D * 2 * KB <= 1024
    float xv = 0.0f;
    int xoff = -1;
    auto load_x = [&](int b) {
        const int t = threadIdx.x;
        xoff = -1;
        if (t < 2 * KB * D) {
            const int mat = t / (KB * D);
            const int rr = (t / D) % KB;
            const int c = t % D;
            const size_t pix = (size_t)slot_pixel(g, w.wy, w.wx, b * KB + rr) * D + c;
            if (mat == 0) {
                xv = dOh[pix];
            } else if constexpr (sizeof(T) == 4) {
                xv = reinterpret_cast<const float*>(Qh)[pix];
            } else {
                xv = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(Qh)[pix] << 16);
            }
            xoff = (mat * KB + rr) * XS + c;
        }
    };

    v4f accV[MTW][NT], accK[MTW][NT];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            accV[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
            accK[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
        }
    load_block(0);
    load_x(0);
    __syncthreads();   // zero fill done

    unsigned cj[EPT];
    for (int b = 0; b < nblk; ++b) {
        // scatter this block's kept entries into the dense planes
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int j = (int)min(ej[u], (unsigned)(N - 1));
            cj[u] = j;
            if (erow[u] >= 0) {
                Md[erow[u] * NP + j] = ea[u];
                Md[(KB + erow[u]) * NP + j] = ek[u];
            }
        }
        if (xoff >= 0) Xs[xoff] = xv;
        __syncthreads();
        if (b + 1 < nblk) {
            load_block(b + 1);
            load_x(b + 1);
        }
        if (wave_active) {
#pragma unroll 1
            for (int ks = 0; ks < KB / 4; ++ks) {
                const int row = 4 * ks + q4;
                float bO[NT], bQ[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    bO[nt] = Xs[row * XS + 16 * nt + r16];
                    bQ[nt] = Xs[(KB + row) * XS + 16 * nt + r16];
                }
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) {
                    if (mt >= mtw) break;
                    const int tile = tile0 + wave * mtw + mt;
                    const float aA = Md[row * NP + 16 * tile + r16];
                    const float aK = Md[(KB + row) * NP + 16 * tile + r16];
                    // SKIP: 4 rows x 16 tokens with no kept entry add nothing (exact for
                    // finite dO and Q); chosen where such sub-blocks are common
                    if (SKIP && __builtin_amdgcn_ballot_w64(aA != 0.0f || aK != 0.0f) == 0) continue;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        accV[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(aA, bO[nt], accV[mt][nt], 0, 0, 0);
                        accK[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(aK, bQ[nt], accK[mt][nt], 0, 0, 0);
                    }
                }
            }
        }
        __syncthreads();
        // reset the slots this thread wrote (the planes are all zero again)
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            if (erow[u] >= 0) {
                Md[erow[u] * NP + cj[u]] = 0.0f;
                Md[(KB + erow[u]) * NP + cj[u]] = 0.0f;
            }
        }
        __syncthreads();
    }
    // lane holds token 16*tile + 4*q4 + r, column 16*nt + r16 of each tile
    if (!wave_active) return;
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
        if (mt >= mtw) break;
        const int tile = tile0 + wave * mtw + mt;
        {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const size_t o = plane + (size_t)slot_pixel(g, w.wy, w.wx, 16 * tile + 4 * q4 + r) * D + r16;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    p.dV[o + 16 * nt] = accV[mt][nt][r];
                    p.dK[o + 16 * nt] = accK[mt][nt][r];
                }
            }
        }
    }
}

template <class F>
hipError_t launch_bwd(F fn, const BackwardArgs& a, int threads, int lds, int grid, hipStream_t s) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(threads), lds, s, a);
    return hipGetLastError();
}

int chunks_per_row(int dtype, int D) { return D * (dtype == 0 ? 4 : 2) / 16; }

// lanes per query row: the smallest of 16, 32, 64 covering ceil(K_l / 4) subgroups
int rows_group(int CH, int K_l) {
    const int need = CH * ((K_l + 3) / 4);
    return need <= 16 ? 16 : need <= 32 ? 32 : 64;
}

int rows_lds(int dtype, int D, int N, int K_l, bool has_v, bool has_k, bool want_dap) {
    const int rowb = D * (dtype == 0 ? 4 : 2);
    const int gl = rows_group(chunks_per_row(dtype, D), K_l);
    const int rsw = (N + 31) / 32 + ((K_l + 3) & ~3);
    return ((has_v ? 1 : 0) + (has_k ? 1 : 0)) * N * rowb +
           ((has_k && want_dap) ? kBwdRowWaves * (64 / gl) * rsw * 4 : 0);
}

template <typename T, int D, bool HV, bool HK>
hipError_t launch_rows_mode(const BackwardArgs& a, int grid, hipStream_t s) {
    constexpr int CH = D * (int)sizeof(T) / 16;
    const int gl = rows_group(CH, a.K_l);
    const int lds = rows_lds(sizeof(T) == 4 ? 0 : 1, D, a.g.N, a.K_l, HV, HK, a.dA_prev != nullptr);
    const int th = kBwdRowWaves * kWave;
    if (gl == 16) return launch_bwd(bwd_rows_kernel<T, D, 16, 1, HV, HK>, a, th, lds, grid, s);
    if (gl == 32) return launch_bwd(bwd_rows_kernel<T, D, 32, 1, HV, HK>, a, th, lds, grid, s);
    const int nst = (a.K_l + 4 * (64 / CH) - 1) / (4 * (64 / CH));
    if (nst <= 1) return launch_bwd(bwd_rows_kernel<T, D, 64, 1, HV, HK>, a, th, lds, grid, s);
    if (nst <= 2) return launch_bwd(bwd_rows_kernel<T, D, 64, 2, HV, HK>, a, th, lds, grid, s);
    if (nst <= 4) return launch_bwd(bwd_rows_kernel<T, D, 64, 4, HV, HK>, a, th, lds, grid, s);
    if constexpr (CH >= 8) {
        if (nst <= 8) return launch_bwd(bwd_rows_kernel<T, D, 64, 8, HV, HK>, a, th, lds, grid, s);
    }
    return hipErrorInvalidValue;   // K_l beyond what the caller admits
}

template <typename T, int D>
hipError_t launch_rows_t(const BackwardArgs& a, bool has_v, bool has_k, int grid, hipStream_t s) {
    if (has_v && has_k) return launch_rows_mode<T, D, true, true>(a, grid, s);
    if (has_v) return launch_rows_mode<T, D, true, false>(a, grid, s);
    return launch_rows_mode<T, D, false, true>(a, grid, s);
}

int scatter_lds(int DH, int N, int K_l) {
    return 2 * N * DH * 4 + kBwdScatterWaves * 3 * ((K_l + 3) & ~3) * 4;
}

int dkv_lds(int D, int N) { return (2 * 16 * (N + 16) + 2 * 16 * (D == 32 ? 48 : 16)) * 4; }

// m-tiles (16 tokens) per wave: a divisor of N/16 that needs at most 16 waves
int dkv_tiles_per_wave(int N) {
    const int mtiles = N / 16;
    for (int mtw = 1; mtw <= 4; mtw *= 2)
        if (mtiles % mtw == 0 && mtiles <= 16 * mtw) return mtw;
    return 0;
}

template <typename T, int D, int EPT, bool SKIP>
hipError_t launch_dkv_e(const BackwardArgs& a, int grid, hipStream_t s) {
    const int th = 16 * kWave;
    const int lds = dkv_lds(D, a.g.N);
    switch (dkv_tiles_per_wave(a.g.N)) {
        case 1: return launch_bwd(bwd_dkv_kernel<T, D, EPT, 1, SKIP>, a, th, lds, grid, s);
        case 2: return launch_bwd(bwd_dkv_kernel<T, D, EPT, 2, SKIP>, a, th, lds, grid, s);
        case 4: return launch_bwd(bwd_dkv_kernel<T, D, EPT, 4, SKIP>, a, th, lds, grid, s);
        default: return hipErrorInvalidValue;   // rejected by backward_dkv_mfma
    }
}

template <typename T, int D>
hipError_t launch_dkv_t(const BackwardArgs& a, int grid, hipStream_t s) {
    const int ept = (16 * a.K_l + 1023) / 1024;
    // all-zero 4 x 16 operand blocks are skipped at a kept density of 1/32 or less
    // (random kept sets: 13 % of the blocks at 1/32, 36 % at 1/64; the test costs
    // 4-5 % at 1/4 and 1/8)
    if (ept <= 1) {
        if (32 * a.K_l <= a.g.N) return launch_dkv_e<T, D, 1, true>(a, grid, s);
        return launch_dkv_e<T, D, 1, false>(a, grid, s);
    }
    if (ept <= 2) return launch_dkv_e<T, D, 2, false>(a, grid, s);
    if (ept <= 4) return launch_dkv_e<T, D, 4, false>(a, grid, s);
    return hipErrorInvalidValue;   // K_l beyond what the caller admits
}

template <typename T, int D>
hipError_t launch_scatter_t(const BackwardArgs& a, int grid, hipStream_t s) {
    const int th = kBwdScatterWaves * kWave;
    if (a.blocks_per_wh == 1)
        return launch_bwd(bwd_scatter_kernel<T, D, D>, a, th, scatter_lds(D, a.g.N, a.K_l), grid, s);
    if (a.blocks_per_wh == 2)
        return launch_bwd(bwd_scatter_kernel<T, D, D / 2>, a, th, scatter_lds(D / 2, a.g.N, a.K_l), grid, s);
    return launch_bwd(bwd_scatter_kernel<T, D, D / 4>, a, th, scatter_lds(D / 4, a.g.N, a.K_l), grid, s);
}

}  // namespace

int backward_fused_rows(int dtype, int D, int N, int K_l, bool want_dap) {
    // one kernel when K and V fit in LDS together and G stays within registers
    // (at most 16 kept slots per lane)
    const int CH = chunks_per_row(dtype, D);
    const int per_lane = 4 * ((K_l + 4 * (64 / CH) - 1) / (4 * (64 / CH)));
    if (per_lane > 16) return 0;
    return rows_lds(dtype, D, N, K_l, true, true, want_dap) <= kLdsBytes ? 1 : 0;
}

bool backward_dkv_mfma(int D, int N, int K_l) {
    return N % 16 == 0 && N <= 1024 && K_l <= 256 && dkv_tiles_per_wave(N) > 0 && dkv_lds(D, N) <= kLdsBytes;
}

int64_t backward_dkv_full(int64_t n_wh, int N, int cus) {
    // one workgroup per CU (its LDS); split only the window-heads of a partial last
    // round, into pairs of halves that fit that round
    if (cus < 16 || dkv_tiles_per_wave(N) % 2 != 0 || n_wh < cus) return n_wh;
    const int64_t full = (n_wh / cus) * cus;
    const int64_t rem = n_wh - full;
    if (rem == 0 || rem % 8 != 0 || 2 * rem > cus || full % 8 != 0) return n_wh;
    return full;
}

hipError_t launch_backward_dkv(const BackwardArgs& a, int dtype, int D, int grid, hipStream_t stream) {
    if (dtype == 0)
        return D == 16 ? launch_dkv_t<float, 16>(a, grid, stream) : launch_dkv_t<float, 32>(a, grid, stream);
    return D == 16 ? launch_dkv_t<uint16_t, 16>(a, grid, stream) : launch_dkv_t<uint16_t, 32>(a, grid, stream);
}

int backward_scatter_parts(int D, int N, int K_l) {
    for (int parts = 1; parts <= 4; parts *= 2)
        if (scatter_lds(D / parts, N, K_l) <= kLdsBytes) return parts;
    return 0;
}

hipError_t launch_backward_rows(const BackwardArgs& a, int dtype, int D, bool has_v, bool has_k, int grid,
                                hipStream_t stream) {
    if (rows_lds(dtype, D, a.g.N, a.K_l, has_v, has_k, a.dA_prev != nullptr) > kLdsBytes) return hipErrorInvalidValue;
    if (dtype == 0)
        return D == 16 ? launch_rows_t<float, 16>(a, has_v, has_k, grid, stream)
                       : launch_rows_t<float, 32>(a, has_v, has_k, grid, stream);
    return D == 16 ? launch_rows_t<uint16_t, 16>(a, has_v, has_k, grid, stream)
                   : launch_rows_t<uint16_t, 32>(a, has_v, has_k, grid, stream);
}

hipError_t launch_backward_scatter(const BackwardArgs& a, int dtype, int D, int grid, hipStream_t stream) {
    if (dtype == 0)
        return D == 16 ? launch_scatter_t<float, 16>(a, grid, stream) : launch_scatter_t<float, 32>(a, grid, stream);
    return D == 16 ? launch_scatter_t<uint16_t, 16>(a, grid, stream) : launch_scatter_t<uint16_t, 32>(a, grid, stream);
}

}  // namespace pfa
