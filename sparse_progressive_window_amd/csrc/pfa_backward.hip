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
//   dA^{l-1}_ir = exp(s_ir) / sum_kept A^{l-1} exp(s) * g_ir  at kept slots, 0 at
//                 dropped ones; this is dkey_ir / A^{l-1}_ir wherever A^l_ir and
//                 A^{l-1}_ir are normal floats (the usual case).
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
//   both passes run in one kernel, keeping G in registers. A row with a kept
//   slot whose A^l or A^{l-1} is zero or subnormal (allowed: a slot of weight 0
//   is kept when K_l exceeds the row's positive weights) has no usable ratio
//   there. Such a slot's A^l is zero or subnormal too (A^l = A^{l-1} exp(s) /
//   sum, with a subnormal A^{l-1} and a normal A^l the true value overflows
//   fp32 anyway), so the K pass flags its workgroup, by A^l, in the workspace.
// * bwd_exact_dap_kernel (after the row pass, only with dA^{l-1}): in flagged
//   workgroups, for each row with such a slot, the log normaliser C = log2 sum_kept A^{l-1} 2^{s2} from the
//   scores themselves (s2 = s log2(e), k_j read from global memory), then
//   dA^{l-1} = 2^{s2 - C} g at the flagged slots. Rare by construction; out of
//   the row kernels, whose registers it would otherwise take.
// * bwd_dkv_kernel (N a multiple of 16, K_l > N / 16): dV = A^T dO and dK = (A g)^T Q / sqrt(d)
//   as dense fp32 MFMA products over row blocks densified in LDS, the dV / dK
//   tiles of each wave's tokens held in registers. At the densities of the keep
//   schedule (K_l / N from 1/4 down to 1/64) this beats accumulating through
//   LDS: on gfx950 an LDS fp32 atomic add retires at ~190 clocks per wavefront
//   instruction and a compare-and-swap loop still costs tens.
// * bwd_dkv_sorted_kernel (K_l <= N / 16, or N not a multiple of 16): the same
//   products with work in proportion to the kept pairs: per row chunk the kept
//   entries are counting-sorted by token in LDS and each token's owner thread
//   sums its records (see the kernel). Deterministic: the sort is keyed by the
//   row, not by arrival.
#include <float.h>

#include "pfa_kernels.h"
#include "pfa_rows.h"

namespace pfa {
namespace {

constexpr int kBwdRowWaves = 16;

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

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <typename T, int D>
__device__ __forceinline__ void load_row_chunk(const T* row, int chunk, float (&o)[Chunk<T>::kElems]) {
    Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(reinterpret_cast<const unsigned char*>(row) + chunk * 16), o);
}

// GLOB (global mode with more than 1024 tokens): k_j and v_j are gathered from
// global memory (L2) instead of the staged window; both passes in one kernel.
template <typename T, int D, int GL, int NST, bool HAS_V, bool HAS_K, bool GLOB = false>
__global__ __launch_bounds__(kBwdRowWaves * kWave) void bwd_rows_kernel(const BackwardArgs p) {
    static_assert(!GLOB || (HAS_V && HAS_K), "global gathers: one kernel");
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

    const unsigned char* Vs;
    const unsigned char* Ks;
    if constexpr (GLOB) {
        Vs = reinterpret_cast<const unsigned char*>(static_cast<const T*>(p.V) + plane);
        Ks = reinterpret_cast<const unsigned char*>(static_cast<const T*>(p.K) + plane);
    } else {
        Vs = smem;
        Ks = smem + (HAS_V ? N * ROWB : 0);
    }
    const int staged = GLOB ? 0 : (HAS_V + HAS_K) * N * ROWB;
    const bool want_dap = HAS_K && p.dA_prev != nullptr;
    const int bmw = (N + 31) >> 5;                       // bitmap words per row
    const int rsw = bmw + ((K_l + 3) & ~3);              // row scratch words
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(smem + staged) + (wave * RPW + grp) * rsw;
    float* vals = reinterpret_cast<float*>(bitmap + bmw);
    // workgroup flag for the exact dA^{l-1} pass, after the row scratch
    uint32_t* wg_flag = reinterpret_cast<uint32_t*>(smem + staged) + NW * RPW * rsw;
    if (want_dap && threadIdx.x == 0) *wg_flag = 0u;
    // smallest A^l over this lane's kept entries of all its rows, as fp32 bits (A^l >= 0
    // orders like its bits): one v_min_u32 per entry, one workgroup flag at the end
    uint32_t amin = 0xFFFFFFFFu;
    if constexpr (!GLOB) {
        if (HAS_V) stage_rows<T, D>(smem, ROWB, static_cast<const T*>(p.V) + plane, g, w.wy, w.wx);
        if (HAS_K) stage_rows<T, D>(smem + (HAS_V ? N * ROWB : 0), ROWB, static_cast<const T*>(p.K) + plane, g, w.wy,
                                    w.wx);
    }
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
                        amin = min(amin, __float_as_uint(av[x]));
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
                        // (a kept slot with A^{l-1} = 0 has A^l = 0 as well: such rows are
                        // flagged from A^l below and rewritten by the exact pass)
                        float val = 0.0f;
                        if (kept && rank < K_l && ap[u] > 0.0f) val = vals[rank] * __builtin_amdgcn_rcpf(ap[u]);
                        if (active && sv) p.dA_prev[srow + slot] = val;
                    }
                }
            }
        }
    }
    if (want_dap) {
        // some kept A^l of this workgroup's rows below FLT_MIN (idle groups looked at
        // row0, one of its rows): the exact pass revisits the workgroup's rows
        if (ballot(amin < 0x00800000u) != 0 && lane == 0) atomicOr(wg_flag, 1u);
        __syncthreads();
        if (threadIdx.x == 0) p.row_flags[blockIdx.x] = (int32_t)*wg_flag;
    }
}

// Exact dA^{l-1} in the workgroups the row pass flagged (one workgroup here per
// row-pass workgroup, same rows). Each wavefront takes rows of the part; a row
// whose kept A^l are all normal floats is skipped, for the others (the lanes
// together):
//   C = log2 sum over kept r with A^{l-1}_r > 0 of A^{l-1}_r 2^{s2_r}  (a running
//       (max, sum) per lane, then over the wave), s2_r = q_i.k_j log2(e) / sqrt(d);
//   dA^{l-1} = 2^{s2_r - C} g_r at the kept slots where A^l_r or A^{l-1}_r is zero
//   or subnormal (the others keep the row pass's dkey / A^{l-1}).
// The kept entry r of I^l (token j) sits at the slot of j in the row's I^{l-1},
// found through a token -> slot table in LDS. q_i and k_j come from global
// memory at the layer's pixels (rare rows: no staging). With a relative position
// bias, s2_r includes the bias of the pair's offset (in base 2).
template <typename T, int D>
__global__ __launch_bounds__(4 * kWave) void bwd_exact_dap_kernel(const BackwardArgs p) {
    constexpr int EPC = Chunk<T>::kElems;
    constexpr int CH = D / EPC;
    __shared__ int16_t pos_all[4][1024];
    if (p.row_flags[blockIdx.x] == 0) return;   // uniform: the usual case
    const Geom g = p.g;
    const int N = g.N;
    const int K_prev = p.K_prev, K_l = p.K_l;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int16_t* pos = pos_all[wave];
    const WhPart w = decode_block(p.blocks_per_wh, p.xcd_map, g);
    const size_t plane = (size_t)w.bh * g.H * g.W * D;
    const T* Qh = static_cast<const T*>(p.Q) + plane;
    const T* Kh = static_cast<const T*>(p.K) + plane;
    const int row0 = w.part * p.rows_per_block;
    const int row1 = min(N, row0 + p.rows_per_block);
    constexpr float kLog2eB = 1.4426950408889634f;
    const float* bt = p.bias ? p.bias + (size_t)(w.bh % g.heads) * (2 * g.win - 1) * (2 * g.win - 1) : nullptr;
    for (int i = row0 + wave; i < row1; i += 4) {
        const size_t row = (size_t)w.wh * N + i;
        const int32_t* Il = p.I_l + row * K_l;
        const float* Al = p.A_l + row * K_l;
        bool low = false;
        for (int e = lane; e < K_l; e += kWave) low |= !(Al[e] >= FLT_MIN);
        if (ballot(low) == 0) continue;
        float qf[D];
#pragma unroll
        for (int c = 0; c < CH; ++c)
            Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(Qh + (size_t)slot_pixel(g, w.wy, w.wx, i) * D + c * EPC),
                             &qf[c * EPC]);
        const int iy = bt ? i / g.win : 0;   // (a bias comes with window mode only)
        const int ibase = (iy + g.win - 1) * (2 * g.win - 1) + (i - iy * g.win) + g.win - 1;
        auto score2 = [&](int j) {
            const T* kr = Kh + (size_t)slot_pixel(g, w.wy, w.wx, j) * D;
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                float kf[EPC];
                Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(kr + c * EPC), kf);
#pragma unroll
                for (int y = 0; y < EPC; ++y) acc = fmaf(qf[c * EPC + y], kf[y], acc);
            }
            if (!bt) return acc * p.scale2;
            const int jy = j / g.win;   // + the bias of the pair's offset, in base 2
            return fmaf(bt[ibase - jy * (2 * g.win - 1) - (j - jy * g.win)], kLog2eB, acc * p.scale2);
        };
        const int32_t* Ip = p.I_prev ? p.I_prev + row * K_prev : nullptr;
        const float* Ap = p.A_prev + row * K_prev;
        const float* Gl = p.g_buf + row * K_l;
        const bool table = Ip && N <= 1024;
        if (table) {
            for (int c = lane; c < K_prev; c += kWave) pos[min((unsigned)Ip[c], (unsigned)(N - 1))] = (int16_t)c;
            __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's table writes before its reads
        }
        // slot of token j in the row's I^{l-1}: the LDS table, or (global mode beyond
        // 1024 tokens, short lists) a search of the row
        auto slot_of = [&](int j) {
            if (!Ip) return j;
            if (table) return (int)pos[j];
            for (int c = 0; c < K_prev; ++c)
                if (Ip[c] == j) return c;
            return 0;   // not a candidate: excluded by the caller's contract
        };
        float mx = -INFINITY, sz = 0.0f;
        for (int e = lane; e < K_l; e += kWave) {
            const int j = (int)min((unsigned)Il[e], (unsigned)(N - 1));
            const float a = Ap[slot_of(j)];
            if (a > 0.0f) {
                const float kap = score2(j) + log2f(a);
                if (kap > mx) {
                    sz = sz * exp2f(mx - kap) + 1.0f;
                    mx = kap;
                } else {
                    sz += exp2f(kap - mx);
                }
            }
        }
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const float mo = __shfl_xor(mx, o);
            const float so = __shfl_xor(sz, o);
            const float mn = fmaxf(mx, mo);
            sz = (mx == -INFINITY ? 0.0f : sz * exp2f(mx - mn)) + (mo == -INFINITY ? 0.0f : so * exp2f(mo - mn));
            mx = mn;
        }
        const float C = mx + log2f(sz);
        for (int e = lane; e < K_l; e += kWave) {
            const int j = (int)min((unsigned)Il[e], (unsigned)(N - 1));
            const int c = slot_of(j);
            const float a = Ap[c];
            if (!(a >= FLT_MIN) || !(Al[e] >= FLT_MIN)) p.dA_prev[row * K_prev + c] = exp2f(score2(j) - C) * Gl[e];
        }
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // table reads done before the next row's writes
    }
}

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

// dK or dV with work in proportion to the kept pairs. A unit is a window-head and
// up to 1024 of its tokens (global mode: several units per head, each taking the
// entries of its token range); each unit has two workgroups, one for dV and one
// for dK, 8 workgroup ids apart so that both run on one XCD and share the unit's
// entries in its L2. Thread t owns token tok0 + t and keeps its row of the
// workgroup's matrix in registers. The window-head's rows are taken in chunks of
// R = 32 MW rows:
//   (a) the chunk's rows of dO (dV) or Q (dK) are staged in LDS (16-byte chunks
//       permuted by row, so the owners' reads of random rows spread over the banks);
//   (b) every kept entry (row r, token j) of the chunk sets bit r of token j's
//       R-bit row mask (LDS or: no order dependence);
//   (c) the masks' popcounts are scanned over the tokens (wave scans, then the
//       wave totals), giving each token a segment of the record list;
//   (d) entry (r, j) is written to its token's segment at the rank of r in j's
//       mask: records come out sorted by token, then by row, whatever the
//       scheduling, so the sums below always run in the same order;
//   (e) each owner adds A dO_r to its dV row, or A g / sqrt(d) q_r to its dK row,
//       over its segment, while the next chunk's entries and rows are loaded.
// Per chunk there are about R K_l / N records per token; the work of the owners
// is K_l d MACs per row, not N d.
template <typename T, int D, int MW>
__global__ __launch_bounds__(16 * kWave) void bwd_dkv_sorted_kernel(const BackwardArgs p) {
    constexpr int R = 32 * MW;                 // rows per chunk
    constexpr int NT = 16 * kWave;             // threads (tokens owned: the first NTK)
    constexpr int EPC = Chunk<T>::kElems;
    constexpr int QCH = D / EPC;               // 16-byte chunks of a Q row
    constexpr int OCH = D / 4;                 // 16-byte chunks of a dO row (fp32)
    constexpr int QROWB = D * (int)sizeof(T);
    constexpr int OROWB = D * 4;
    constexpr int EPT = 8192 / NT;             // entries per thread (the launcher keeps R K_l <= 8192)
    constexpr int RL = (R * OCH + NT - 1) / NT;   // 16-byte row chunks per thread
    extern __shared__ __align__(16) unsigned char smem[];

    const int xcd = (int)blockIdx.x & 7;
    const int slot = (int)blockIdx.x >> 3;
    const bool kmat = (slot & 1) != 0;         // false: dV, true: dK (uniform)
    const int unit = (slot >> 1) * 8 + xcd;
    if (unit >= p.dkv_units) return;           // padding of the last group of 8 units

    const Geom g = p.g;
    const int N = g.N;   // rows (and tokens) of the window-head
    const int K_l = p.K_l;
    const unsigned kmagic = (unsigned)((0x100000000ull + (unsigned)K_l - 1u) / (unsigned)K_l);   // ceil(2^32 / K_l)
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wave = t / kWave;
    const int tparts = (N + NT - 1) / NT;
    const int tok0 = (unit % tparts) * NT;   // this workgroup's tokens: [tok0, tok0 + NTK)
    const int NTK = min(NT, N - tok0);
    const WhPart w = decode_block_id(unit / tparts, 1, p.xcd_map, g);
    const size_t plane = (size_t)w.bh * g.H * g.W * D;
    const unsigned char* Qh = reinterpret_cast<const unsigned char*>(static_cast<const T*>(p.Q) + plane);
    const unsigned char* dOh = reinterpret_cast<const unsigned char*>(p.dO + plane);

    unsigned char* rows = smem;                                       // [R][OROWB]: dO or Q rows
    uint32_t* mask = reinterpret_cast<uint32_t*>(rows + R * OROWB);   // [MW][NTK]: word m of token j at m NTK + j
    int* seg = reinterpret_cast<int*>(mask + NTK * MW);               // [NTK] segment starts
    int* wsum = seg + NTK;                                            // [16] wave totals
    const size_t roff = ((size_t)(R * OROWB + (NTK * MW + NTK + 16) * 4) + 7) & ~(size_t)7;
    float* recw = reinterpret_cast<float*>(smem + roff);              // [R K_l] A, or A g / sqrt(d)
    uint16_t* recr = reinterpret_cast<uint16_t*>(recw + R * K_l);     // [R K_l] row in the chunk

    const size_t wh_pairs = (size_t)w.wh * N * K_l;
    const int pair_bytes = N * K_l * 4;
    const __amdgpu_buffer_rsrc_t rI = make_rsrc(p.I_l + wh_pairs, pair_bytes);
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A_l + wh_pairs, pair_bytes);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.g_buf + wh_pairs, pair_bytes);

    // a chunk's rows and entries (raw), loaded one chunk ahead
    int ej[EPT];
    float ea[EPT], eg[EPT];
    uint4 rr[RL];
    auto load_chunk = [&](int r0) {
        const int rows_c = min(R, N - r0);
        const int ne = rows_c * K_l;
        // rows first: their addresses may need a reloaded value, whose wait must not
        // also wait for the entries
        if (kmat) {
#pragma unroll
            for (int k = 0; k < RL; ++k) {
                const int u = t + NT * k;
                if (u < rows_c * QCH) {
                    const int r = u / QCH, c = u - r * QCH;
                    rr[k] = *reinterpret_cast<const uint4*>(Qh + (size_t)slot_pixel(g, w.wy, w.wx, r0 + r) * QROWB +
                                                            c * 16);
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < RL; ++k) {
                const int u = t + NT * k;
                if (u < rows_c * OCH) {
                    const int r = u / OCH, c = u - r * OCH;
                    rr[k] = *reinterpret_cast<const uint4*>(dOh + (size_t)slot_pixel(g, w.wy, w.wx, r0 + r) * OROWB +
                                                            c * 16);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            int e = t + NT * u;
            __asm__ volatile("" : "+v"(e));
            const int off = e < ne ? (r0 * K_l + e) * 4 : 0x7FFFFFF0;   // past the range: not loaded
            ej[u] = (int)__builtin_amdgcn_raw_buffer_load_b32(rI, off, 0, 0);
            ea[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rA, off, 0, 0));
            if (kmat) eg[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, off, 0, 0));
        }
    };
    float acc[D];
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] = 0.0f;

    load_chunk(0);
    if (t < NTK) {
#pragma unroll
        for (int m = 0; m < MW; ++m) mask[m * NTK + t] = 0u;   // (the owners clear them again after each chunk)
    }
    __syncthreads();   // every mask is clear before any entry of the first chunk is set
    for (int r0 = 0; r0 < N; r0 += R) {
        const int rows_c = min(R, N - r0);
        const int ne = rows_c * K_l;
        // (a) the chunk's rows into LDS (the previous chunk's owners are done)
        if (kmat) {
#pragma unroll
            for (int k = 0; k < RL; ++k) {
                const int u = t + NT * k;
                if (u < rows_c * QCH) {
                    const int r = u / QCH, c = u - r * QCH;
                    *reinterpret_cast<uint4*>(rows + r * QROWB + ((c ^ (r & (QCH - 1))) * 16)) = rr[k];
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < RL; ++k) {
                const int u = t + NT * k;
                if (u < rows_c * OCH) {
                    const int r = u / OCH, c = u - r * OCH;
                    *reinterpret_cast<uint4*>(rows + r * OROWB + ((c ^ (r & (OCH - 1))) * 16)) = rr[k];
                }
            }
        }
        // the entries' tokens (- tok0, or -1: no entry, or another unit's token) and weights
        int jr[EPT];
        float wt[EPT];
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            int e = t + NT * u;
            __asm__ volatile("" : "+v"(e));
            const int j = (int)min((unsigned)ej[u], (unsigned)(N - 1));   // memory safety only: indices lie in [0, N)
            jr[u] = (e < ne && j >= tok0 && j - tok0 < NTK) ? j - tok0 : -1;
            wt[u] = kmat ? ea[u] * eg[u] * p.scale : ea[u];
        }
        // (b) row masks per token. The entry's row r = e / K_l comes from a multiply-high
        // (exact for e < 2^13 and K_l <= 256); e is made opaque per chunk, so that the
        // EPT rows and their masks are not kept live across the chunk loop.
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            int e = t + NT * u;
            __asm__ volatile("" : "+v"(e));
            if (jr[u] >= 0) {
                const int r = (int)__umulhi((unsigned)e, kmagic);
                atomicOr(&mask[(r >> 5) * NTK + jr[u]], 1u << (r & 31));
            }
        }
        __syncthreads();
        // (c) segment of each token: exclusive scan of the mask popcounts
        int cnt = 0;
        if (t < NTK) {
#pragma unroll
            for (int m = 0; m < MW; ++m) cnt += __builtin_popcount(mask[m * NTK + t]);
        }
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        if (lane == kWave - 1) wsum[wave] = incl;
        __syncthreads();
        int base = 0;
        for (int v = 0; v < wave; ++v) base += wsum[v];
        const int st = base + incl - cnt;
        if (t < NTK) seg[t] = st;
        __syncthreads();
        // (d) records at the rank of their row in the token's mask
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            int e = t + NT * u;
            __asm__ volatile("" : "+v"(e));
            if (jr[u] >= 0) {
                const int r = (int)__umulhi((unsigned)e, kmagic);
                const uint32_t* mj = mask + jr[u];
                int rank = __builtin_popcount(mj[(r >> 5) * NTK] & ((1u << (r & 31)) - 1u));
#pragma unroll
                for (int m = 0; m < MW; ++m)
                    if (m < (r >> 5)) rank += __builtin_popcount(mj[m * NTK]);
                const int pos = seg[jr[u]] + rank;
                recw[pos] = wt[u];
                recr[pos] = (uint16_t)r;
            }
        }
        __syncthreads();
        // the next chunk's loads are in flight during the owners' sums
        if (r0 + R < N) load_chunk(r0 + R);
        // (e) owners: their segment in row order; their masks are cleared for the next chunk
        if (t < NTK) {
#pragma unroll
            for (int m = 0; m < MW; ++m) mask[m * NTK + t] = 0u;
        }
        if (kmat) {
            for (int k = st; k < st + cnt; ++k) {
                const float wv = recw[k];
                const int r = recr[k];
#pragma unroll
                for (int c = 0; c < QCH; ++c) {
                    float qf[EPC];
                    Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(rows + r * QROWB + ((c ^ (r & (QCH - 1))) * 16)),
                                     qf);
#pragma unroll
                    for (int y = 0; y < EPC; ++y) acc[EPC * c + y] = fmaf(wv, qf[y], acc[EPC * c + y]);
                }
            }
        } else {
            for (int k = st; k < st + cnt; ++k) {
                const float wv = recw[k];
                const int r = recr[k];
#pragma unroll
                for (int c = 0; c < OCH; ++c) {
                    const float4 o4 = *reinterpret_cast<const float4*>(rows + r * OROWB + ((c ^ (r & (OCH - 1))) * 16));
                    acc[4 * c + 0] = fmaf(wv, o4.x, acc[4 * c + 0]);
                    acc[4 * c + 1] = fmaf(wv, o4.y, acc[4 * c + 1]);
                    acc[4 * c + 2] = fmaf(wv, o4.z, acc[4 * c + 2]);
                    acc[4 * c + 3] = fmaf(wv, o4.w, acc[4 * c + 3]);
                }
            }
        }
        __syncthreads();   // the next chunk reuses the LDS
    }
    if (t < NTK) {
        float* dst = (kmat ? p.dK : p.dV) + plane + (size_t)slot_pixel(g, w.wy, w.wx, tok0 + t) * D;
#pragma unroll
        for (int c = 0; c < D; c += 4)
            *reinterpret_cast<float4*>(dst + c) = make_float4(acc[c], acc[c + 1], acc[c + 2], acc[c + 3]);
    }
}

// The same with both matrices in one workgroup per unit (window-head and 1024
// tokens): thread t owns token tok0 + t and keeps its dV and dK rows in
// registers, with no room left to load the next chunk during the sums. Steps
// (a)-(e) as above, with the chunk's dO and Q rows both staged and records of
// (A, A g / sqrt(d)). Used where the units fill the CUs over several rounds
// anyway, so that splitting the matrices over two workgroups would only repeat
// steps (a)-(d).
template <typename T, int D, int MW>
__global__ __launch_bounds__(16 * kWave) void bwd_dkv_sorted_pair_kernel(const BackwardArgs p) {
    constexpr int R = 32 * MW;                 // rows per chunk
    constexpr int NT = 16 * kWave;             // threads (tokens owned: the first N)
    constexpr int EPC = Chunk<T>::kElems;
    constexpr int QCH = D / EPC;               // 16-byte chunks of a Q row
    constexpr int OCH = D / 4;                 // 16-byte chunks of a dO row (fp32)
    constexpr int QROWB = D * (int)sizeof(T);
    constexpr int OROWB = D * 4;
    extern __shared__ __align__(16) unsigned char smem[];

    const Geom g = p.g;
    const int N = g.N;   // rows (and tokens) of the window-head
    const int K_l = p.K_l;
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wave = t / kWave;
    const int tparts = (N + NT - 1) / NT;
    const int tok0 = (blockIdx.x % tparts) * NT;   // this workgroup's tokens: [tok0, tok0 + NTK)
    const int NTK = min(NT, N - tok0);
    const WhPart w = decode_block_id(blockIdx.x / tparts, 1, p.xcd_map, g);
    const size_t plane = (size_t)w.bh * g.H * g.W * D;
    const T* Qh = static_cast<const T*>(p.Q) + plane;
    const float* dOh = p.dO + plane;

    unsigned char* dOs = smem;                                        // [R][OROWB]
    unsigned char* Qs = dOs + R * OROWB;                              // [R][QROWB]
    uint32_t* mask = reinterpret_cast<uint32_t*>(Qs + R * QROWB);     // [MW][NTK]: word m of token j at m NTK + j
    int* seg = reinterpret_cast<int*>(mask + NTK * MW);               // [NTK] segment starts
    int* wsum = seg + NTK;                                            // [16] wave totals
    const size_t roff = ((size_t)(R * OROWB + R * QROWB + (NTK * MW + NTK + 16) * 4) + 7) & ~(size_t)7;
    float2* recw = reinterpret_cast<float2*>(smem + roff);            // [R K_l] (A, A g / sqrt(d))
    uint16_t* recr = reinterpret_cast<uint16_t*>(recw + R * K_l);     // [R K_l] row in the chunk

    const size_t wh_pairs = (size_t)w.wh * N * K_l;
    const int pair_bytes = N * K_l * 4;
    const __amdgpu_buffer_rsrc_t rI = make_rsrc(p.I_l + wh_pairs, pair_bytes);
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A_l + wh_pairs, pair_bytes);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.g_buf + wh_pairs, pair_bytes);

    float accV[D], accK[D];
#pragma unroll
    for (int c = 0; c < D; ++c) accV[c] = accK[c] = 0.0f;
    constexpr int EPT = 8192 / NT;   // entries per thread (the launcher keeps R K_l <= 8192)

    if (t < NTK) {
#pragma unroll
        for (int m = 0; m < MW; ++m) mask[m * NTK + t] = 0u;   // (the owners clear them again after each chunk)
    }
    for (int r0 = 0; r0 < N; r0 += R) {
        const int rows = min(R, N - r0);
        const int ne = rows * K_l;
        // (a) stage the chunk's rows; load its entries
        for (int u = t; u < rows * OCH; u += NT) {
            const int r = u / OCH, c = u - r * OCH;
            *reinterpret_cast<float4*>(dOs + r * OROWB + ((c ^ (r & (OCH - 1))) * 16)) =
                *reinterpret_cast<const float4*>(dOh + (size_t)slot_pixel(g, w.wy, w.wx, r0 + r) * D + c * 4);
        }
        for (int u = t; u < rows * QCH; u += NT) {
            const int r = u / QCH, c = u - r * QCH;
            *reinterpret_cast<uint4*>(Qs + r * QROWB + ((c ^ (r & (QCH - 1))) * 16)) = *reinterpret_cast<const uint4*>(
                reinterpret_cast<const unsigned char*>(Qh + (size_t)slot_pixel(g, w.wy, w.wx, r0 + r) * D) + c * 16);
        }
        int ej[EPT];   // token - tok0, or -1 (no entry, or another workgroup's token)
        float ea[EPT], ek[EPT];
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = t + NT * u;
            const int off = e < ne ? (r0 * K_l + e) * 4 : 0x7FFFFFF0;   // past the range: not loaded
            const int j = (int)min((unsigned)__builtin_amdgcn_raw_buffer_load_b32(rI, off, 0, 0), (unsigned)(N - 1));
            ej[u] = (e < ne && j >= tok0 && j - tok0 < NTK) ? j - tok0 : -1;
            ea[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rA, off, 0, 0));
            ek[u] = ea[u] * __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, off, 0, 0)) * p.scale;
        }
        __syncthreads();
        // (b) row masks per token
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = t + NT * u;
            if (ej[u] >= 0) {
                const int r = e / K_l;
                atomicOr(&mask[(r >> 5) * NTK + ej[u]], 1u << (r & 31));
            }
        }
        __syncthreads();
        // (c) segment of each token: exclusive scan of the mask popcounts
        int cnt = 0;
        if (t < NTK) {
#pragma unroll
            for (int m = 0; m < MW; ++m) cnt += __builtin_popcount(mask[m * NTK + t]);
        }
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        if (lane == kWave - 1) wsum[wave] = incl;
        __syncthreads();
        int base = 0;
        for (int v = 0; v < wave; ++v) base += wsum[v];
        const int st = base + incl - cnt;
        if (t < NTK) seg[t] = st;
        __syncthreads();
        // (d) records at the rank of their row in the token's mask
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = t + NT * u;
            if (ej[u] >= 0) {
                const int r = e / K_l;
                const uint32_t* mj = mask + ej[u];
                int rank = __builtin_popcount(mj[(r >> 5) * NTK] & ((1u << (r & 31)) - 1u));
#pragma unroll
                for (int m = 0; m < MW; ++m)
                    if (m < (r >> 5)) rank += __builtin_popcount(mj[m * NTK]);
                const int pos = seg[ej[u]] + rank;
                recw[pos] = make_float2(ea[u], ek[u]);
                recr[pos] = (uint16_t)r;
            }
        }
        __syncthreads();
        // (e) owners: their segment in row order; their masks are cleared for the next chunk
        if (t < NTK) {
#pragma unroll
            for (int m = 0; m < MW; ++m) mask[m * NTK + t] = 0u;
        }
        for (int k = st; k < st + cnt; ++k) {
            const float2 wv = recw[k];
            const int r = recr[k];
#pragma unroll
            for (int c = 0; c < OCH; ++c) {
                const float4 o4 = *reinterpret_cast<const float4*>(dOs + r * OROWB + ((c ^ (r & (OCH - 1))) * 16));
                accV[4 * c + 0] = fmaf(wv.x, o4.x, accV[4 * c + 0]);
                accV[4 * c + 1] = fmaf(wv.x, o4.y, accV[4 * c + 1]);
                accV[4 * c + 2] = fmaf(wv.x, o4.z, accV[4 * c + 2]);
                accV[4 * c + 3] = fmaf(wv.x, o4.w, accV[4 * c + 3]);
            }
#pragma unroll
            for (int c = 0; c < QCH; ++c) {
                float qf[EPC];
                Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(Qs + r * QROWB + ((c ^ (r & (QCH - 1))) * 16)), qf);
#pragma unroll
                for (int y = 0; y < EPC; ++y) accK[EPC * c + y] = fmaf(wv.y, qf[y], accK[EPC * c + y]);
            }
        }
        __syncthreads();   // the next chunk reuses the LDS
    }
    if (t < NTK) {
        const size_t o = plane + (size_t)slot_pixel(g, w.wy, w.wx, tok0 + t) * D;
#pragma unroll
        for (int c = 0; c < D; c += 4) {
            *reinterpret_cast<float4*>(p.dV + o + c) = make_float4(accV[c], accV[c + 1], accV[c + 2], accV[c + 3]);
            *reinterpret_cast<float4*>(p.dK + o + c) = make_float4(accK[c], accK[c + 1], accK[c + 2], accK[c + 3]);
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

// global mode with more than 1024 tokens: nothing staged (gathers from L2)
bool rows_global(int N) { return N > 1024; }

int rows_lds(int dtype, int D, int N, int K_l, bool has_v, bool has_k, bool want_dap) {
    const int rowb = D * (dtype == 0 ? 4 : 2);
    const int gl = rows_group(chunks_per_row(dtype, D), K_l);
    const int rsw = (N + 31) / 32 + ((K_l + 3) & ~3);
    const int staged = rows_global(N) ? 0 : ((has_v ? 1 : 0) + (has_k ? 1 : 0)) * N * rowb;
    return staged + ((has_k && want_dap) ? kBwdRowWaves * (64 / gl) * rsw * 4 + 16 : 0);   // + the workgroup flag
}

template <typename T, int D, bool HV, bool HK, bool GLOB>
hipError_t launch_rows_mode(const BackwardArgs& a, int grid, hipStream_t s) {
    constexpr int CH = D * (int)sizeof(T) / 16;
    const int gl = rows_group(CH, a.K_l);
    const int lds = rows_lds(sizeof(T) == 4 ? 0 : 1, D, a.g.N, a.K_l, HV, HK, a.dA_prev != nullptr);
    const int th = kBwdRowWaves * kWave;
    if (gl == 16) return launch_bwd(bwd_rows_kernel<T, D, 16, 1, HV, HK, GLOB>, a, th, lds, grid, s);
    if (gl == 32) return launch_bwd(bwd_rows_kernel<T, D, 32, 1, HV, HK, GLOB>, a, th, lds, grid, s);
    const int nst = (a.K_l + 4 * (64 / CH) - 1) / (4 * (64 / CH));
    if (nst <= 1) return launch_bwd(bwd_rows_kernel<T, D, 64, 1, HV, HK, GLOB>, a, th, lds, grid, s);
    if (nst <= 2) return launch_bwd(bwd_rows_kernel<T, D, 64, 2, HV, HK, GLOB>, a, th, lds, grid, s);
    if (nst <= 4) return launch_bwd(bwd_rows_kernel<T, D, 64, 4, HV, HK, GLOB>, a, th, lds, grid, s);
    if constexpr (CH >= 8) {
        if (nst <= 8) return launch_bwd(bwd_rows_kernel<T, D, 64, 8, HV, HK, GLOB>, a, th, lds, grid, s);
    }
    return hipErrorInvalidValue;   // K_l beyond what the caller admits
}

template <typename T, int D>
hipError_t launch_rows_t(const BackwardArgs& a, bool has_v, bool has_k, int grid, hipStream_t s) {
    if (rows_global(a.g.N)) {
        if (!has_v || !has_k) return hipErrorInvalidValue;   // one kernel in global mode
        return launch_rows_mode<T, D, true, true, true>(a, grid, s);
    }
    if (has_v && has_k) return launch_rows_mode<T, D, true, true, false>(a, grid, s);
    if (has_v) return launch_rows_mode<T, D, true, false, false>(a, grid, s);
    return launch_rows_mode<T, D, false, true, false>(a, grid, s);
}

// rows per chunk of the sorted dK/dV kernel: the largest of 32, 64, 128, 256 rows
// (at most N rounded up to 32) whose LDS (staged rows, token masks, records) fits
// LDS of the sorted dK/dV kernels (staged rows, token masks, records); pair: both
// matrices in one workgroup
int sorted_lds(int dtype, int D, int N, int K_l, int R, bool pair) {
    const int rowb = pair ? D * 4 + D * (dtype == 0 ? 4 : 2) : D * 4;
    const int recb = pair ? 10 : 6;
    const int nt = N < 1024 ? N : 1024;   // tokens per workgroup
    return R * rowb + (nt * (R / 32) + nt + 16) * 4 + 8 + R * K_l * recb;
}

// rows per chunk of the sorted dK/dV kernels: the largest of 32, 64, 128, 256 rows
// (at most N rounded up to 32) whose LDS fits; 0: none fits
int sorted_rows(int dtype, int D, int N, int K_l, bool pair) {
    if (K_l > 256) return 0;
    int best = 0;
    for (int R = 32; R <= 256; R *= 2) {
        if (R * K_l > 8192) break;
        if (sorted_lds(dtype, D, N, K_l, R, pair) <= kLdsBytes) best = R;
        if (R >= N) break;
    }
    return best;
}

template <typename T, int D>
hipError_t launch_sorted_t(const BackwardArgs& a, bool split, int grid, hipStream_t s) {
    constexpr int dt = sizeof(T) == 4 ? 0 : 1;
    const int R = sorted_rows(dt, D, a.g.N, a.K_l, !split);
    const int lds = sorted_lds(dt, D, a.g.N, a.K_l, R, !split);
    const int th = 16 * kWave;
    if (split) {
        switch (R) {
            case 32: return launch_bwd(bwd_dkv_sorted_kernel<T, D, 1>, a, th, lds, grid, s);
            case 64: return launch_bwd(bwd_dkv_sorted_kernel<T, D, 2>, a, th, lds, grid, s);
            case 128: return launch_bwd(bwd_dkv_sorted_kernel<T, D, 4>, a, th, lds, grid, s);
            case 256: return launch_bwd(bwd_dkv_sorted_kernel<T, D, 8>, a, th, lds, grid, s);
            default: return hipErrorInvalidValue;   // rejected by backward_dkv_sorted
        }
    }
    switch (R) {
        case 32: return launch_bwd(bwd_dkv_sorted_pair_kernel<T, D, 1>, a, th, lds, grid, s);
        case 64: return launch_bwd(bwd_dkv_sorted_pair_kernel<T, D, 2>, a, th, lds, grid, s);
        case 128: return launch_bwd(bwd_dkv_sorted_pair_kernel<T, D, 4>, a, th, lds, grid, s);
        case 256: return launch_bwd(bwd_dkv_sorted_pair_kernel<T, D, 8>, a, th, lds, grid, s);
        default: return hipErrorInvalidValue;   // the caller checks sorted_rows first
    }
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

}  // namespace

int backward_fused_rows(int dtype, int D, int N, int K_l, bool want_dap) {
    // one kernel when K and V fit in LDS together and G stays within registers
    // (at most 16 kept slots per lane)
    // (global mode beyond 1024 tokens gathers both from L2: always one kernel)
    const int CH = chunks_per_row(dtype, D);
    const int per_lane = 4 * ((K_l + 4 * (64 / CH) - 1) / (4 * (64 / CH)));
    if (rows_global(N)) return 1;
    if (per_lane > 16) return 0;
    return rows_lds(dtype, D, N, K_l, true, true, want_dap) <= kLdsBytes ? 1 : 0;
}

bool backward_dkv_sorted(int dtype, int D, int N, int K_l) {
    // measured on the MI355X (fp32 and bf16, N = 1024, both matrices in one
    // workgroup): per window-head about 90 us of fixed cost (chunk loads and
    // barriers, one workgroup per CU) plus 2.5 us per kept slot of a row; the dense
    // MFMA form costs about N^2 whatever K_l. The sorted form wins from K_l = N / 16
    // down (0.66 against 1.53 ms at K_l = 16 on the 640x384 map, 1.48 against 1.87
    // at K_l = 64, 4.0 against 2.2 at K_l = 256), and it is the only form for N not
    // a multiple of 16 when it fits
    if (sorted_rows(dtype, D, N, K_l, false) == 0) return false;
    return 16 * K_l <= N || !backward_dkv_mfma(D, N, K_l);
}

bool backward_dkv_sorted_split(int dtype, int D, int N, int K_l, int64_t units, int cus) {
    // one workgroup per CU either way (1024 threads at 128 VGPRs). A one-matrix
    // workgroup takes 0.51-0.59 of a two-matrix one (its next chunk loads during the
    // sums), so the split pays where it needs fewer than about 1.8 times the rounds:
    // 384 window-heads on 256 CUs (3 rounds against 2), not 1440 (12 against 6)
    if (sorted_rows(dtype, D, N, K_l, true) == 0) return true;
    if (cus <= 0) return false;
    const int64_t pair_rounds = (units + cus - 1) / cus;
    const int64_t split_rounds = (2 * units + cus - 1) / cus;
    return split_rounds * 11 < pair_rounds * 20;
}

hipError_t launch_backward_dkv_sorted(const BackwardArgs& a, int dtype, int D, bool split, int grid,
                                      hipStream_t stream) {
    if (dtype == 0)
        return D == 16 ? launch_sorted_t<float, 16>(a, split, grid, stream)
                       : launch_sorted_t<float, 32>(a, split, grid, stream);
    return D == 16 ? launch_sorted_t<uint16_t, 16>(a, split, grid, stream)
                   : launch_sorted_t<uint16_t, 32>(a, split, grid, stream);
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

hipError_t launch_backward_rows(const BackwardArgs& a, int dtype, int D, bool has_v, bool has_k, int grid,
                                hipStream_t stream) {
    if (rows_lds(dtype, D, a.g.N, a.K_l, has_v, has_k, a.dA_prev != nullptr) > kLdsBytes) return hipErrorInvalidValue;
    if (dtype == 0)
        return D == 16 ? launch_rows_t<float, 16>(a, has_v, has_k, grid, stream)
                       : launch_rows_t<float, 32>(a, has_v, has_k, grid, stream);
    return D == 16 ? launch_rows_t<uint16_t, 16>(a, has_v, has_k, grid, stream)
                   : launch_rows_t<uint16_t, 32>(a, has_v, has_k, grid, stream);
}

hipError_t launch_backward_exact_dap(const BackwardArgs& a, int dtype, int D, int grid, hipStream_t stream) {
    auto go = [&](auto fn) {
        hipLaunchKernelGGL(fn, dim3(grid), dim3(4 * kWave), 0, stream, a);
        return hipGetLastError();
    };
    if (dtype == 0) return D == 16 ? go(bwd_exact_dap_kernel<float, 16>) : go(bwd_exact_dap_kernel<float, 32>);
    return D == 16 ? go(bwd_exact_dap_kernel<uint16_t, 16>) : go(bwd_exact_dap_kernel<uint16_t, 32>);
}

}  // namespace pfa
