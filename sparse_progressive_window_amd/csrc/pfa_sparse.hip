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
// staging. A query row is handled by a group of GL lanes (GL = 4 .. 64, with KPT
// candidates per lane, GL*KPT >= K_prev, both picked by the launcher from K_prev;
// a wavefront handles 64/GL rows at once); lane l of the group owns candidates
// c = l + GL*t (coalesced loads of
// the I^{l-1} / A^{l-1} rows). k_j is gathered from LDS reading the 16-byte
// chunks of the row in a lane-rotated order, so 8 consecutive lanes always touch
// 8 different chunks and a 128-byte row never bank-conflicts.
//
// Top-K. Keys are the fp32 bit patterns of u (u >= 0, so integer order = float
// order). The K_l-th largest key is found exactly by radix descent: the current
// key interval is split into GL bit-field bins counted with LDS atomics, a DPP
// prefix scan over the bins (descending) locates the bin holding the K_l-th key,
// and the search recurses into it; keys in higher bins are kept, lower ones are
// dropped. Reductions inside a group use DPP (quad permutes, row rotations, row
// broadcasts), ds_swizzle for the 16-lane half swap and readlane across halves.
// Exact ties at the threshold keep the lowest slot indices (bisection on j).
//
// Kept entries are compacted in I^{l-1} order (ballot + lane-prefix counts) and
// staged in LDS as (j, weight); the aggregation then gives each V row chunk to
// a lane (CH lanes read one whole row, conflict-free) and sums the lanes of a
// group with row rotations.
#include <type_traits>

#include "pfa_kernels.h"
#include "pfa_rows.h"

namespace pfa {
namespace {


typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));


struct MaxF { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct SumF { __device__ float operator()(float a, float b) const { return a + b; } };
struct MaxI { __device__ int operator()(int a, int b) const { return max(a, b); } };
struct MinI { __device__ int operator()(int a, int b) const { return min(a, b); } };
struct SumI { __device__ int operator()(int a, int b) const { return a + b; } };

// Reductions and counts over a group of GL consecutive lanes (GL = 4 .. 64); every
// lane of the group receives the result.
template <int GL>
struct Grp {
    static_assert(GL == 4 || GL == 8 || GL == 16 || GL == 32 || GL == 64, "group width");
    template <class Op>
    __device__ static float all(float v, Op op) {
        v = op(v, dppf<kQuadXor1>(v));
        v = op(v, dppf<kQuadXor2>(v));
        if (GL == 8) v = op(v, dppf<kRowHalfMirror>(v));   // the other quad of the 8-lane half
        if (GL >= 16) {
            v = op(v, dppf<kRowRor4>(v));
            v = op(v, dppf<kRowRor8>(v));
        }
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
        if (GL == 8) v = op(v, dpp<kRowHalfMirror>(v));
        if (GL >= 16) {
            v = op(v, dpp<kRowRor4>(v));
            v = op(v, dpp<kRowRor8>(v));
        }
        if (GL >= 32) v = op(v, swap16(v));
        if (GL == 64) v = op(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 32));
        return v;
    }
    static constexpr int kLog2 = GL == 64 ? 6 : GL == 32 ? 5 : GL == 16 ? 4 : GL == 8 ? 3 : 2;
    // inclusive prefix sum over the lanes of the group (row_shr steps, then row
    // broadcasts across the 16-lane rows; narrower groups mask the steps that would
    // reach into the previous group)
    __device__ static unsigned incl_scan(unsigned x) {
        if (GL < 16) {
            const unsigned l = __lane_id() & (GL - 1);
            unsigned y = (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
            x += l >= 1 ? y : 0u;
            y = (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);            // row_shr:2
            x += l >= 2 ? y : 0u;
            if (GL == 8) {
                y = (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);        // row_shr:4
                x += l >= 4 ? y : 0u;
            }
            return x;
        }
        x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
        x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
        x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
        x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
        if (GL >= 32) x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
        if (GL == 64) x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
        return x;
    }
    // lanes of this lane's group as a wave mask
    __device__ static uint64_t group_mask(int lane) {
        if (GL == 64) return ~0ull;
        return ((1ull << GL) - 1ull) << (lane & (64 - GL));
    }
    // bits of the wave mask m that belong to this lane's group
    __device__ static uint32_t bits(uint64_t m, int lane) {
        if (GL == 64) return 0;  // unused
        const uint32_t half = (lane & 32) ? (uint32_t)(m >> 32) : (uint32_t)m;
        if (GL == 32) return half;
        return (half >> (lane & (32 - GL))) & ((1u << GL) - 1u);
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


// sum the lanes of a group that own the same chunk (lane bits [log2 CH, log2 GL))
template <int CH, int GL>
__device__ __forceinline__ float reduce_chunk_lanes(float v) {
    if (GL <= 8) {
        // groups narrower than a 16-lane DPP row: xor exchanges stay inside the group
        // (a row rotate would pull lanes of the neighbouring group)
        if (CH <= 1 && GL >= 2) v += dppf<kQuadXor1>(v);
        if (CH <= 2 && GL >= 4) v += dppf<kQuadXor2>(v);
        if (CH <= 4 && GL >= 8) v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F));  // xor 4
        return v;
    }
    if (CH <= 2) v += dppf<kRowRor2>(v);
    if (CH <= 4 && GL >= 8) v += dppf<kRowRor4>(v);
    if (CH <= 8 && GL >= 16) v += dppf<kRowRor8>(v);
    if (GL >= 32) v += swap16f(v);
    if (GL == 64) v += __shfl_xor(v, 32);
    return v;
}

// Where a row's V vectors come from in a fused aggregation (global mode: the
// raster rows of the map), or none.
enum VSrc { kVraster = 0, kVnone = 1 };

// u = A^{l-1} exp(s - m) for one query row held by a group of GL lanes, in place
// over the base-2 scores sv (m = the row maximum). fmaxf maps NaN and negative
// products (invalid previous maps) to 0, so keys always lie in [0, +inf] and
// every search in select_emit terminates.
template <int GL, int KPT>
__device__ __forceinline__ void keys_from_scores(const float (&av)[KPT], const bool (&valid)[KPT],
                                                 float (&sv)[KPT]) {
    float smax = -INFINITY;
#pragma unroll
    for (int t = 0; t < KPT; ++t) smax = fmaxf(smax, sv[t]);
    smax = Grp<GL>::all(smax, MaxF());
#pragma unroll
    for (int t = 0; t < KPT; ++t) sv[t] = valid[t] ? fmaxf(av[t] * fast_exp2(sv[t] - smax), 0.0f) : 0.0f;
}

// Exact K_l-th largest key of one query row held by a group of GL lanes (key(t)
// = this lane's t-th key, -1 for no candidate) by radix descent: the key
// interval [lo, hi) is cut into NB = BPL*GL bins of 2^shift consecutive keys
// (bit-field slices), counted with LDS atomics; a prefix scan over the bins in
// descending order (BPL bins per lane) finds the bin that holds the K_l-th key;
// keys in higher bins are kept, keys in lower bins are dropped, and the search
// descends into that bin. Each level removes log2(NB) bits from the interval, so
// it ends after at most 8 levels (usually 2 or 3). Result: every key > tau is
// kept, need_tau more are needed among the n_tau keys equal to tau.
// RES0: the level's result (bin, count above, count in bin) is passed through
// words 0..2 of the histogram itself (their counts have been read by then)
// instead of three words past its end.
template <int GL, int BPL, int KPT, bool RES0 = false, class KF>
__device__ __forceinline__ void radix_threshold(KF key, int kmin, int kmax, bool active, int K_prev, int K_l,
                                                unsigned* hb, int gl, int& tau, int& need_tau, int& n_tau) {
    using G = Grp<GL>;
    constexpr int NB = BPL * GL;
    constexpr int RES = RES0 ? 0 : NB;
    constexpr int LOG2NB = G::kLog2 + (BPL == 8 ? 3 : BPL == 4 ? 2 : BPL == 2 ? 1 : 0);
    static_assert(BPL == 1 || BPL == 2 || BPL == 4 || BPL == 8, "bins per lane");
    int lo = kmin, hi = kmax + 1, need = K_l;
    tau = lo;
    need_tau = K_l;
    n_tau = 0;
    bool done = !active;
    if (active && hi - lo <= 1) {   // all keys equal
        done = true;
        n_tau = K_prev;
    }
    while (ballot(!done) != 0) {
        const int span = max(hi - lo, 2);
        const int shift = max(32 - __clz(span - 1) - LOG2NB, 0);
        if (BPL >= 4) {
#pragma unroll
            for (int b = 0; b < BPL; b += 4) {
                // zeros made here (a zero quad kept live across the caller's loop was spilled)
                unsigned z;
                __asm__ volatile("v_mov_b32 %0, 0" : "=v"(z));
                *reinterpret_cast<uint4*>(hb + BPL * gl + b) = make_uint4(z, z, z, z);
            }
        } else if (BPL == 2) {
            *reinterpret_cast<uint2*>(hb + 2 * gl) = make_uint2(0u, 0u);
        } else {
            hb[gl] = 0u;
        }
#pragma unroll
        for (int t = 0; t < KPT; ++t) {
            const unsigned dk = (unsigned)(key(t) - lo);
            if (!done && dk < (unsigned)(hi - lo)) atomicAdd(&hb[dk >> shift], 1u);
        }
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // this lane's bins in descending key order: NB-1-BPL*gl-b, b = 0..BPL-1
        unsigned cb[BPL];
        if (BPL >= 4) {
#pragma unroll
            for (int b = 0; b < BPL; b += 4) {
                const uint4 c4 = *reinterpret_cast<const uint4*>(hb + NB - BPL * (gl + 1) + b);
                cb[BPL - 1 - b] = c4.x;
                cb[BPL - 2 - b] = c4.y;
                cb[BPL - 3 - b] = c4.z;
                cb[BPL - 4 - b] = c4.w;
            }
        } else if (BPL == 2) {
            const uint2 c2 = *reinterpret_cast<const uint2*>(hb + NB - 2 - 2 * gl);
            cb[0] = c2.y;
            cb[BPL - 1] = c2.x;
        } else {
            cb[0] = hb[NB - 1 - gl];
        }
        unsigned lsum = 0;
#pragma unroll
        for (int b = 0; b < BPL; ++b) lsum += cb[b];
        const unsigned incl = G::incl_scan(lsum);
        unsigned run = incl - lsum;
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
            if (!done && run < (unsigned)need && run + cb[b] >= (unsigned)need) {   // exactly one bin per group
                hb[RES] = (unsigned)(NB - 1 - BPL * gl - b);
                hb[RES + 1] = run;
                hb[RES + 2] = cb[b];
            }
            run += cb[b];
        }
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int bin = (int)hb[RES];
        const int above = (int)hb[RES + 1];
        const int in_bin = (int)hb[RES + 2];
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (!done) {
            need -= above;
            lo += bin << shift;
            hi = min(hi, lo + (1 << shift));
            if (in_bin == need || hi - lo <= 1) {   // whole bin kept, or all its keys equal (ties)
                tau = lo;
                need_tau = need;
                n_tau = in_bin;
                done = true;
            }
        }
    }
}

// Exact ties at the threshold keep the lowest slot indices: the smallest jcut
// such that need_tau keys equal to tau have j <= jcut (bisection on j), or
// INT_MAX when the row has no tie to break. any_tie: some row of the wave has.
template <int GL, int KPT, class KF, class JF>
__device__ __forceinline__ int tie_cut(KF key, JF jf, int tau, int need_tau, int n_tau, bool active, int N,
                                       bool& any_tie) {
    using G = Grp<GL>;
    int jcut = 0x7fffffff;
    const bool tie = active && n_tau > need_tau;
    any_tie = ballot(tie) != 0;
    if (any_tie) {
        int jl = -1, jh = N - 1;
        while (ballot(tie && jh - jl > 1) != 0) {
            const int mid = (jl + jh) >> 1;
            // a copy of tau made inside the loop keeps the KPT comparisons from being
            // hoisted out of it as KPT live lane masks
            int tq = tau, mq = mid;
            __asm__ volatile("" : "+v"(tq), "+v"(mq));
            int cl = 0;   // per-lane count, then one group sum
#pragma unroll
            for (int t = 0; t < KPT; ++t) cl += (key(t) == tq && jf(t) <= mq) ? 1 : 0;
            const int cnt = G::all_i(cl, SumI());
            if (tie && jh - jl > 1) {
                if (cnt >= need_tau) jh = mid; else jl = mid;
            }
        }
        if (tie) jcut = jh;
    }
    return jcut;
}

// Everything after the keys of one query row: the exact top-K_l (ties to the
// lower slot index), the I^l / A^l row in I^{l-1} order and, unless
// VS == kVnone, O_i = sum_kept A v_j. jj/valid/uv are this lane's candidates
// c = gl + GL*t; uv = A^{l-1} exp(s - m) >= 0.
template <typename T, int D, int GL, int KPT, int VS, int BPL>
__device__ __forceinline__ void select_emit(const SparseArgs& p, const Geom& g, int lane, bool active, size_t row,
                                            int qpix, const int (&jj)[KPT], const bool (&valid)[KPT],
                                            const float (&uv_in)[KPT], unsigned* hb, uint2* scr, int scg,
                                            const T* Vh, float* Oh) {
    constexpr int EPC = Chunk<T>::kElems;
    constexpr int CH = D / EPC;
    constexpr int GS = GL / CH;
    using G = Grp<GL>;
    const int gl = lane & (GL - 1);
    const int K_prev = p.K_prev;
    const int K_l = p.K_l;

    float uv[KPT];
    int key[KPT];
    int kmin = 0x7fffffff, kmax = -1;
#pragma unroll
    for (int t = 0; t < KPT; ++t) {
        uv[t] = uv_in[t];
        key[t] = valid[t] ? __float_as_int(uv[t]) : -1;
        if (valid[t]) {
            kmin = min(kmin, key[t]);
            kmax = max(kmax, key[t]);
        }
    }
    kmin = G::all_i(kmin, MinI());
    kmax = G::all_i(kmax, MaxI());

    int tau, need_tau, n_tau;
    radix_threshold<GL, BPL, KPT>([&](int t) { return key[t]; }, kmin, kmax, active, K_prev, K_l, hb, gl, tau,
                                  need_tau, n_tau);
    bool tie;
    const int jcut = tie_cut<GL, KPT>([&](int t) { return key[t]; }, [&](int t) { return jj[t]; }, tau, need_tau,
                                      n_tau, active, g.N, tie);

    bool kept[KPT];
    float ksum = 0.0f;
    if (!tie) {   // usual case: every key equal to tau is kept
#pragma unroll
        for (int t = 0; t < KPT; ++t) kept[t] = key[t] >= tau;
    } else {
#pragma unroll
        for (int t = 0; t < KPT; ++t) kept[t] = key[t] > tau || (key[t] == tau && jj[t] <= jcut);
    }
#pragma unroll
    for (int t = 0; t < KPT; ++t) ksum += kept[t] ? uv[t] : 0.0f;
    const float inv = 1.0f / G::all(ksum, SumF());

    // kept entries in I^{l-1} order: positions by ballot prefix counts, staged in
    // LDS as (j, weight), then written as contiguous row segments
    int pos[KPT];
    int obase = 0;
#pragma unroll
    for (int t = 0; t < KPT; ++t) {
        const uint64_t m = ballot(kept[t]);
        pos[t] = kept[t] ? obase + G::below(m, lane) : -1;
        if (pos[t] >= K_l) pos[t] = -1;   // only on precondition violations
        uv[t] *= inv;
        obase += G::count_mask(m, lane);
    }
    int32_t* Io = p.I_out + row * K_l;
    float* Ao = p.A_out + row * K_l;
    const int vchunk = gl % CH;
    const int vsub = gl / CH;
    float oacc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) oacc[e] = 0.0f;
    for (int P0 = 0; P0 < K_l; P0 += scg) {
#pragma unroll
        for (int t = 0; t < KPT; ++t)
            if (pos[t] >= P0 && pos[t] < P0 + scg)
                scr[pos[t] - P0] = make_uint2((uint32_t)jj[t], __float_as_uint(uv[t]));
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int cnt = active ? min(scg, K_l - P0) : 0;
        for (int e = gl; e < cnt; e += GL) {
            const uint2 ent = scr[e];
            Io[P0 + e] = (int32_t)ent.x;
            Ao[P0 + e] = __uint_as_float(ent.y);
        }
        if (VS != kVnone) {
            // O_i = sum_kept A v_j: CH lanes read one V row; GS entries at a time per group
            for (int e = vsub; e < cnt; e += GS) {
                const uint2 ent = scr[e];
                const float w = __uint_as_float(ent.y);
                const unsigned char* vrow = reinterpret_cast<const unsigned char*>(Vh + (size_t)ent.x * D);
                float vf[EPC];
                Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(vrow + vchunk * 16), vf);
#pragma unroll
                for (int x = 0; x < EPC; ++x) oacc[x] = fmaf(w, vf[x], oacc[x]);
            }
        }
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    if (VS == kVnone) return;
#pragma unroll
    for (int x = 0; x < EPC; ++x) oacc[x] = reduce_chunk_lanes<CH, GL>(oacc[x]);
    if (active && vsub == 0) {
        float* orow = Oh + (size_t)qpix * D + vchunk * EPC;
#pragma unroll
        for (int x = 0; x < EPC; x += 4)
            *reinterpret_cast<float4*>(orow + x) = make_float4(oacc[x], oacc[x + 1], oacc[x + 2], oacc[x + 3]);
    }
}

// Top-K_l of one query row held by a group of GL lanes, written straight from
// registers (no aggregation in this kernel): lane gl's t-th candidate is slot
// jf(t), present when vf(t), with weight uv[t] = A^{l-1} exp(s - m) >= 0. The
// kept entries of register t occupy consecutive positions across the group's
// lanes (ballot prefix counts), so the t-loop emits I^l / A^l in candidate order
// with one store per register through buffer resources (32-bit offsets).
// ORDERED: jf is increasing in (t, lane) order, so exact ties at the threshold
// are resolved by rank in that order (the lowest slots first) within the store
// loop; otherwise by bisection on j.
struct NoHook {
    __device__ void operator()() const {}
};

// pre_store runs once the selection is done with the histogram words, before the
// store loop (the all-candidates kernel puts its next batch's query rows there).
template <int GL, int KPT, int BPL, bool ORDERED, bool RES0 = false, class JF, class VF, class PS = NoHook>
__device__ __forceinline__ void select_store(const SparseArgs& p, int lane, bool active, int N, JF jf, VF vf,
                                             const float (&uv)[KPT], unsigned* hb, __amdgpu_buffer_rsrc_t rI,
                                             __amdgpu_buffer_rsrc_t rA, int row_off, PS pre_store = PS()) {
    using G = Grp<GL>;
    const int gl = lane & (GL - 1);
    const int K_prev = p.K_prev;
    const int K_l = p.K_l;
    auto key = [&](int t) { return vf(t) ? __float_as_int(uv[t]) : -1; };

    int kmin = 0x7fffffff, kmax = -1;
#pragma unroll
    for (int t = 0; t < KPT; ++t) {
        if (vf(t)) {
            kmin = min(kmin, key(t));
            kmax = max(kmax, key(t));
        }
    }
    kmin = G::all_i(kmin, MinI());
    kmax = G::all_i(kmax, MaxI());

    int tau, need_tau, n_tau;
    radix_threshold<GL, BPL, KPT, RES0>(key, kmin, kmax, active, K_prev, K_l, hb, gl, tau, need_tau, n_tau);
    // tie: more keys equal tau (the interval shrank to one key value) than are needed
    const bool tie = active && n_tau > need_tau;
    const bool any_tie = ballot(tie) != 0;
    int jcut = 0x7fffffff;
    if (!ORDERED && any_tie) {
        bool unused;
        jcut = tie_cut<GL, KPT>(key, jf, tau, need_tau, n_tau, active, N, unused);
    }

    // kept = key > thr, plus (ties) some keys equal to tau: thr = tau - 1 keeps every
    // key equal to tau; on an ORDERED tie row thr = tau and the tied keys are added
    // by rank below (they all weigh u_tau)
    const int thr = (ORDERED && tie) ? tau : tau - 1;
    float ksum = 0.0f;
    if (!ORDERED && any_tie) {
#pragma unroll
        for (int t = 0; t < KPT; ++t) ksum += (key(t) > tau || (key(t) == tau && jf(t) <= jcut)) ? uv[t] : 0.0f;
    } else {
#pragma unroll
        for (int t = 0; t < KPT; ++t) ksum += key(t) > thr ? uv[t] : 0.0f;
    }
    ksum = G::all(ksum, SumF());
    if (ORDERED && tie) ksum += (float)need_tau * __int_as_float(tau);
    const float inv = 1.0f / ksum;
    pre_store();

    // Store loop. Positions: group-masked ballots counted with mbcnt, the running
    // group count folded into the accumulator. Entries not to be stored (not kept,
    // rows past the end) get an offset past the buffer resource's range, which the
    // hardware drops. The descent keeps exactly K_l entries of an active row, so
    // positions stay below K_l; only the bisection tie cut can keep more (repeated
    // indices in I^{l-1}, a precondition violation), where positions past K_l are
    // dropped too. The loop
    // compares with copies of thr/tau the compiler cannot see through, so it does
    // not keep KPT comparison masks alive from the sums above.
    int thr2 = thr, tau2 = tau;
    __asm__ volatile("" : "+v"(thr2), "+v"(tau2));
    const uint64_t gmask = G::group_mask(lane);
    const uint32_t gm_lo = (uint32_t)gmask, gm_hi = (uint32_t)(gmask >> 32);
    int obase = 0;
    int tbase = 0;   // ORDERED ties: keys equal to tau met so far in the group
    auto emit = [&](int t, bool k, bool guard) {
        const uint64_t m = ballot(k);
        const uint32_t ml = (uint32_t)m & gm_lo, mh = (uint32_t)(m >> 32) & gm_hi;
        // pos is made opaque so that the offset stays a select, not a branch
        int pos = (int)__builtin_amdgcn_mbcnt_hi(mh, __builtin_amdgcn_mbcnt_lo(ml, (uint32_t)obase));
        __asm__ volatile("" : "+v"(pos));
        const int off = (k && (!guard || pos < K_l)) ? (row_off + pos) * 4 : 0x7FFFFFF0;
        __builtin_amdgcn_raw_buffer_store_b32(jf(t), rI, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(uv[t] * inv), rA, off, 0, 0);
        // two accumulating bit counts (v_bcnt_u32_b32 adds its second operand)
        int part = __builtin_popcount(ml) + obase;
        __asm__ volatile("" : "+v"(part));
        obase = __builtin_popcount(mh) + part;
    };
    if (!any_tie) {
#pragma unroll
        for (int t = 0; t < KPT; ++t) emit(t, key(t) > thr2, false);
    } else if (ORDERED) {
#pragma unroll
        for (int t = 0; t < KPT; ++t) {
            const bool eq = tie && key(t) == tau2;
            const uint64_t me = ballot(eq);
            const int rank = tbase + G::below(me, lane);
            tbase += G::count_mask(me, lane);
            emit(t, key(t) > thr2 || (eq && rank < need_tau), false);
        }
    } else {
#pragma unroll
        for (int t = 0; t < KPT; ++t) emit(t, key(t) > tau2 || (key(t) == tau2 && jf(t) <= jcut), true);
    }
}


// Generic sparse layer: scores by LDS (or global) gathers of k_j, one group of GL
// lanes per query row.
// FULL: K_prev == GL*KPT, so every candidate slot of an active row exists (no
// per-candidate validity), scores stay raw until the exponent; inactive row
// groups of the last iteration are scored on row0's data and never stored.
// BIAS (window mode): the head's relative position bias b[(dy + w - 1)(2w - 1) +
// dx + w - 1] of (i, j) is added to the scaled score; the (2w - 1)^2-entry table
// is read through a range-checked buffer resource (it stays in L1), because at
// fp32 d = 32 the staged K rows and the histograms fill the LDS.
template <typename T, int D, int GL, int KPT, int MODE, int NW, bool PQ, bool FULL, bool BIAS = false>
__global__ __launch_bounds__(NW * kWave) void sparse_layer_kernel(const SparseArgs p) {
    constexpr int EPC = Chunk<T>::kElems;   // elements per 16-byte chunk
    constexpr int CH = D / EPC;             // chunks per K/V row
    constexpr int ROWB = D * (int)sizeof(T);
    constexpr int RPW = kWave / GL;         // rows per wavefront iteration
    constexpr bool K_LDS = MODE == kKselect;
    constexpr int VS = MODE == kKVglobal ? kVraster : kVnone;
    constexpr int BPL = VS == kVnone ? 4 : 1;        // radix bins per lane (no (j, weight) staging: more bins)
    constexpr int HISTG = BPL * GL + 4;              // histogram words per row group
    constexpr int HISTW = RPW * HISTG;               // radix-select histogram words per wave
    constexpr int HIST_BYTES = NW * HISTW * 4;
    static_assert(HIST_BYTES <= kScratchBytes, "histograms exceed the scratch area");
    constexpr int SCW = VS == kVnone ? 0 : (kScratchBytes - HIST_BYTES) / (NW * 8);   // (j, weight) entries per wave
    constexpr int SCG = SCW / RPW;                                                   // entries per row group
    extern __shared__ __align__(16) unsigned char smem[];

    const Geom g = p.g;
    const int N = g.N;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int grp = lane / GL;
    const int gl = lane & (GL - 1);
    const WhPart w = decode_block(p.blocks_per_wh, p.xcd_map, g);
    const size_t plane = (size_t)w.bh * g.H * g.W * D;
    const T* Qh = static_cast<const T*>(p.Q) + plane;
    const T* Kh = static_cast<const T*>(p.K) + plane;
    const T* Vh = static_cast<const T*>(p.V) + plane;
    float* Oh = p.O_out + plane;

    unsigned char* Ks = smem;
    unsigned char* sbase = smem + (K_LDS ? N * ROWB : 0);
    unsigned* hb = reinterpret_cast<unsigned*>(sbase) + wave * HISTW + grp * HISTG;
    uint2* scr = reinterpret_cast<uint2*>(sbase + HIST_BYTES) + wave * SCW + grp * SCG;


    int coff[CH];   // lane-rotated chunk order for whole-row gathers
#pragma unroll
    for (int m = 0; m < CH; ++m) coff[m] = ((m + lane) % CH) * 16;

    const int row0 = w.part * p.rows_per_block;
    const int row1 = min(N, row0 + p.rows_per_block);
    const int K_prev = p.K_prev;

    // Software pipeline over the wavefront's rows: the global loads of the next
    // row (candidate list, previous weights and, when PQ, the query vector) are in
    // flight while the current row is scored and selected.
    struct RowIn {
        int j[KPT];
        float a[KPT];
        uint4 q[PQ ? CH : 1];
    };
    auto load_row = [&](RowIn& r, int base) {
        const int i_raw = base + grp;
        const bool active = i_raw < row1;
        const int i = active ? i_raw : row0;
        const size_t row = (size_t)w.wh * N + i;
        const size_t rowI = p.i_shared ? (size_t)(w.b * w.nwin + w.win_id) * N + i : row;
        const int32_t* Irow = p.I_prev ? p.I_prev + rowI * K_prev + gl : nullptr;
        const float* Arow = p.A_prev ? p.A_prev + row * K_prev + gl : nullptr;
        if (FULL) {
            // the weights of a FULL row are loaded after its scores (late_a)
#pragma unroll
            for (int t = 0; t < KPT; ++t) r.j[t] = Irow ? Irow[GL * t] : gl + GL * t;
        } else {
#pragma unroll
            for (int t = 0; t < KPT; ++t) {
                const int c = gl + GL * t;
                const bool v = active && c < K_prev;
                r.j[t] = v ? (Irow ? Irow[GL * t] : c) : 0;
                r.a[t] = (v && Arow) ? Arow[GL * t] : 1.0f;
            }
        }
        if (PQ) {
            const unsigned char* qrow =
                reinterpret_cast<const unsigned char*>(Qh + (size_t)slot_pixel(g, w.wy, w.wx, i) * D);
#pragma unroll
            for (int m = 0; m < CH; ++m) r.q[m] = *reinterpret_cast<const uint4*>(qrow + coff[m]);
        }
    };
    // QS: the query rows of the wave's next batch are loaded before this batch's
    // I/A stores (loads issued after them would wait for them too: one in-order
    // counter) and pass through the wave's histogram words, free between selections
    // (measured 4-8 % faster with 8 candidates per lane, neutral or slower with fewer)
    constexpr bool QS = !PQ && VS == kVnone && KPT >= 8 && ROWB / 4 <= HISTG;
    constexpr int QW = RPW * ROWB / 4;                 // words of the batch's query rows
    constexpr int NQ = (QW + kWave - 1) / kWave;
    static_assert(!QS || QW <= HISTW, "query rows exceed the histogram words");
    unsigned* qst = reinterpret_cast<unsigned*>(sbase) + wave * HISTW;
    auto load_qs = [&](int b0, unsigned (&qd)[NQ]) {
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const int u = lane + kWave * k;
            qd[k] = 0u;
            if (u < QW) {
                const int r = u / (ROWB / 4);
                const int ir = b0 + r;
                const int iq = ir < row1 ? ir : row0;
                const unsigned* qrow = reinterpret_cast<const unsigned*>(Qh + (size_t)slot_pixel(g, w.wy, w.wx, iq) * D);
                qd[k] = qrow[u - r * (ROWB / 4)];
            }
        }
    };
    auto put_qs = [&](const unsigned (&qd)[NQ]) {
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const int u = lane + kWave * k;
            if (u < QW) qst[u] = qd[k];
        }
    };
    // the first rows' loads go out before the window's K is staged, so their
    // latency overlaps the staging
    unsigned qd0[NQ];
    if constexpr (QS) load_qs(row0 + wave * RPW, qd0);
    RowIn cur;
    load_row(cur, row0 + wave * RPW);
    if (K_LDS) {
        stage_rows<T, D>(Ks, ROWB, Kh, g, w.wy, w.wx);
        __syncthreads();
    }
    if constexpr (QS) put_qs(qd0);
    for (int base = row0 + wave * RPW; base < row1; base += NW * RPW) {
        RowIn nxt;
        if (base + NW * RPW < row1) load_row(nxt, base + NW * RPW);
        const int i_raw = base + grp;
        const bool active = i_raw < row1;
        const int i = active ? i_raw : row0;
        const int qpix = slot_pixel(g, w.wy, w.wx, i);
        const size_t row = (size_t)w.wh * N + i;

        int jj[KPT];
        bool valid[KPT];
#pragma unroll
        for (int t = 0; t < KPT; ++t) {
            valid[t] = FULL || (active && gl + GL * t < K_prev);
            jj[t] = (int)min((unsigned)cur.j[t], (unsigned)(N - 1));   // memory safety only: indices lie in [0, N)
        }

        // the query row: fp32 values, or for bf16 the packed pairs themselves (v_dot2c_f32_bf16
        // multiplies the bf16 pairs exactly and accumulates in fp32, like the fp32 FMA chain)
        constexpr bool DOT2 = sizeof(T) == 2;
        float qf[DOT2 ? 1 : D];
        uint4 qp[DOT2 ? CH : 1];
        {
            const unsigned char* qrow = reinterpret_cast<const unsigned char*>(Qh + (size_t)qpix * D);
#pragma unroll
            for (int m = 0; m < CH; ++m) {
                const uint4 c = PQ   ? cur.q[m]
                                : QS ? *reinterpret_cast<const uint4*>(reinterpret_cast<const unsigned char*>(qst) +
                                                                        grp * ROWB + coff[m])
                                     : *reinterpret_cast<const uint4*>(qrow + coff[m]);
                if constexpr (DOT2) qp[m] = c;
                else Chunk<T>::to_f32(c, &qf[m * EPC]);
            }
        }

        // relative position bias of (i, j_t) in base-2 units, loads issued before the scores
        float b2[BIAS ? KPT : 1];
        if constexpr (BIAS) {
            const int nrel = (2 * g.win - 1) * (2 * g.win - 1);
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.bias + (size_t)(w.bh % g.heads) * nrel, nrel * 4);
            const int iy = (i * g.win_magic) >> 16;
            const int ibase = (iy + g.win - 1) * (2 * g.win - 1) + (i - iy * g.win) + g.win - 1;
#pragma unroll
            for (int t = 0; t < KPT; ++t) {
                const int jy = (jj[t] * g.win_magic) >> 16;
                const int idx = ibase - jy * (2 * g.win - 1) - (jj[t] - jy * g.win);
                b2[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, idx * 4, 0, 0));
            }
#pragma unroll
            for (int t = 0; t < KPT; ++t) b2[t] *= 1.4426950408889634f;
        }

        // SMM: scores over the candidate list only (base-2 units)
        float sv[KPT];
#pragma unroll
        for (int t = 0; t < KPT; ++t) {
            const unsigned char* krow =
                K_LDS ? Ks + jj[t] * ROWB : reinterpret_cast<const unsigned char*>(Kh + (size_t)jj[t] * D);
            float acc = 0.0f;
#pragma unroll
            for (int m = 0; m < CH; ++m) {
                const uint4 kc = *reinterpret_cast<const uint4*>(krow + coff[m]);
                if constexpr (DOT2) {
                    acc = dot2_bf16(qp[m].x, kc.x, acc);
                    acc = dot2_bf16(qp[m].y, kc.y, acc);
                    acc = dot2_bf16(qp[m].z, kc.z, acc);
                    acc = dot2_bf16(qp[m].w, kc.w, acc);
                } else {
                    float kf[EPC];
                    Chunk<T>::to_f32(kc, kf);
#pragma unroll
                    for (int e = 0; e < EPC; ++e) acc = fmaf(qf[m * EPC + e], kf[e], acc);
                }
            }
            if constexpr (BIAS)
                sv[t] = (FULL || valid[t]) ? fmaf(acc, p.scale2, b2[t]) : -INFINITY;
            else
                sv[t] = FULL ? acc : (valid[t] ? acc * p.scale2 : -INFINITY);
        }
        if (FULL && BIAS) {
            // scores already scaled and biased: u = A^{l-1} exp2(s - max s)
            float smax = sv[0];
#pragma unroll
            for (int t = 1; t < KPT; ++t) smax = fmaxf(smax, sv[t]);
            const float c = -Grp<GL>::all(smax, MaxF());
            const float* Arow = p.A_prev ? p.A_prev + row * K_prev + gl : nullptr;
            float a[KPT];
#pragma unroll
            for (int t = 0; t < KPT; ++t) a[t] = Arow ? Arow[GL * t] : 1.0f;
#pragma unroll
            for (int t = 0; t < KPT; ++t) sv[t] = fmaxf(a[t] * fast_exp2(sv[t] + c), 0.0f);
        } else if (FULL) {
            // u = A^{l-1} exp2(scale2 (s - max s)); fmaxf maps invalid previous weights to 0.
            // A^{l-1} is loaded only now: no prefetched weights occupy registers
            // during the scoring (the other waves of the SIMD cover the latency)
            float smax = sv[0];
#pragma unroll
            for (int t = 1; t < KPT; ++t) smax = fmaxf(smax, sv[t]);
            const float c = -Grp<GL>::all(smax, MaxF()) * p.scale2;
            const float* Arow = p.A_prev ? p.A_prev + row * K_prev + gl : nullptr;
            float a[KPT];
            if (Arow) {
#pragma unroll
                for (int t = 0; t < KPT; ++t) a[t] = Arow[GL * t];
            } else {
#pragma unroll
                for (int t = 0; t < KPT; ++t) a[t] = 1.0f;
            }
#pragma unroll
            for (int t = 0; t < KPT; ++t) sv[t] = fmaxf(a[t] * fast_exp2(fmaf(sv[t], p.scale2, c)), 0.0f);
        } else {
            keys_from_scores<GL, KPT>(cur.a, valid, sv);
        }
        if constexpr (VS == kVnone) {
            const size_t rbase = ((size_t)w.wh * N + base) * p.K_l;
            const int nbytes = max(0, min(RPW, row1 - base)) * p.K_l * 4;
            unsigned qn[NQ];
            const bool more = base + NW * RPW < row1;
            if (QS && more) load_qs(base + NW * RPW, qn);
            select_store<GL, KPT, BPL, false>(
                p, lane, active, N, [&](int t) { return jj[t]; }, [&](int t) { return FULL || valid[t]; }, sv, hb,
                make_rsrc(p.I_out + rbase, nbytes), make_rsrc(p.A_out + rbase, nbytes), grp * p.K_l);
            if (QS && more) put_qs(qn);
        } else {
            select_emit<T, D, GL, KPT, VS, BPL>(p, g, lane, active, row, qpix, jj, valid, sv, hb, scr, SCG, Vh,
                                                Oh);
        }
        cur = nxt;
    }
}

// MFMA operand helpers for the all-candidates layer: 16 independent 4x4 blocks;
// lane l feeds row l%4 of block l/4 in the A operand and column l%4 of block l/4
// in the B operand, and receives D[block][r][l%4] in accumulator register r.
template <typename T>
struct Mfma4;

// chunk(a, b, c): c += the products of one 16-byte chunk of a query row (a) and
// of a K row (b), as they sit in memory
template <>
struct Mfma4<float> {
    __device__ static v4f chunk(const uint4 a, const uint4 b, v4f c) {
        c = __builtin_amdgcn_mfma_f32_4x4x1f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_4x4x1f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_4x4x1f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_4x4x1f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    }
};

template <>
struct Mfma4<uint16_t> {
    // a 16-byte chunk holds 8 bf16 values: two operands of 4 for 4x4x4 (element e
    // of an operand is bits 16e..16e+15 of the pair of dwords, as in memory)
    __device__ static v4f chunk(const uint4 a, const uint4 b, v4f c) {
        c = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(v4s, make_uint2(a.x, a.y)),
                                                   __builtin_bit_cast(v4s, make_uint2(b.x, b.y)), c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(v4s, make_uint2(a.z, a.w)),
                                                      __builtin_bit_cast(v4s, make_uint2(b.z, b.w)), c, 0, 0, 0);
    }
};

// Chunk permutation of the LDS-resident K rows of the all-candidates kernel
// (128- or 64-byte rows, no pad): chunk c of row r is stored at position
// c ^ kswz(r), so the MFMA operand reads of 16 consecutive rows at one chunk
// position touch 16 different 16-byte bank groups (and 8 consecutive rows 8).
template <int CH>
__device__ __forceinline__ int kswz(int r) {
    if (CH == 8) return (r ^ (r >> 3)) & 7;
    return (r ^ (r >> 2)) & 3;
}

// Reduction of one value per row for the 4 rows of a wave whose values are spread
// over all 64 lanes (v[r] = this lane's part of row r): a swap across the 32-lane
// halves and a swap across 16-lane rows pair the rows up (v_permlane32_swap,
// v_permlane16_swap), then a 16-lane reduction. Row g's result ends in every lane
// of the 16-lane group g.
template <class Op>
__device__ __forceinline__ float rows4_to_groups(const float (&v)[4], Op op) {
    const auto p02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[2]), false, false);
    const auto p13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[1]), __float_as_uint(v[3]), false, false);
    const float w02 = op(__uint_as_float(p02[0]), __uint_as_float(p02[1]));   // rows 0 | 2
    const float w13 = op(__uint_as_float(p13[0]), __uint_as_float(p13[1]));   // rows 1 | 3
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(w02), __float_as_uint(w13), false, false);
    return Grp<16>::all(op(__uint_as_float(q[0]), __uint_as_float(q[1])), op);
}
template <class Op>
__device__ __forceinline__ int rows4_to_groups_i(const int (&v)[4], Op op) {
    const auto p02 = __builtin_amdgcn_permlane32_swap((unsigned)v[0], (unsigned)v[2], false, false);
    const auto p13 = __builtin_amdgcn_permlane32_swap((unsigned)v[1], (unsigned)v[3], false, false);
    const int w02 = op((int)p02[0], (int)p02[1]);
    const int w13 = op((int)p13[0], (int)p13[1]);
    const auto q = __builtin_amdgcn_permlane16_swap((unsigned)w02, (unsigned)w13, false, false);
    return Grp<16>::all_i(op((int)q[0], (int)q[1]), op);
}

// Selection-only layer whose candidate list is every slot of a 32x32 window
// (I^{l-1} implicit, K_prev = N = 1024). Scores of a batch of 4 query rows x 64
// candidates come from 4x4 MFMA blocks (A = the 4 query rows, B = 64 K rows from
// LDS), which leaves candidate 64t + l of all 4 rows in lane l. The selection
// works in that layout: each row's keys span the whole wave, the 4 rows' radix
// levels share their LDS round trips, and only the bin scans run one row per
// 16-lane group.
// DUAL: fused first two layers; the scores are q1.k1 + q.k (the first layer's Q/K
// under shift1 as a second K region in LDS), with no previous map: by the
// closed form of the chain, the second layer keeps the top K_l of
// A^1 (.) softmax(s2), i.e. of exp(s1 + s2) up to a row constant.
template <typename T, int D, bool HAS_A, bool DUAL>
__global__ __launch_bounds__(16 * kWave) void all_cand_rows_kernel(const SparseArgs p) {
    constexpr int NW = 16;
    constexpr int GL = 16;                   // lanes that scan one row's bins
    constexpr int BPL = 8;                   // 128 radix bins per row
    constexpr int EPC = Chunk<T>::kElems;
    constexpr int CH = D / EPC;
    constexpr int ROWB = D * (int)sizeof(T);
    constexpr bool SWZ = CH == 8 || CH == 4;   // 128- and 64-byte rows: chunk-swizzled, unpadded
    constexpr int NK = DUAL ? 2 : 1;            // K regions in LDS
    constexpr int KSTR = SWZ ? ROWB : ROWB + 16;
    constexpr int HISTG = BPL * GL;       // the level results reuse words 0..2
    extern __shared__ __align__(16) unsigned char smem[];

    const Geom g = p.g;
    const int N = g.N;   // 1024
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const WhPart w = decode_block(p.blocks_per_wh, p.xcd_map, g);
    const size_t plane = (size_t)w.bh * g.H * g.W * D;
    const T* Qh = static_cast<const T*>(p.Q) + plane;
    const T* Kh = static_cast<const T*>(p.K) + plane;

    Geom g1 = g;   // DUAL: the first layer's slot geometry
    g1.shift = p.shift1;
    const T* Q1h = DUAL ? static_cast<const T*>(p.Q1) + plane : nullptr;
    const T* K1h = DUAL ? static_cast<const T*>(p.K1) + plane : nullptr;

    unsigned char* Ks = smem;
    unsigned* hist0 = reinterpret_cast<unsigned*>(smem + NK * N * KSTR);
    auto stage_k = [&](unsigned char* dst, const T* src_plane, const Geom& gg) {
        if (SWZ) {
            for (int u = threadIdx.x; u < N * CH; u += blockDim.x) {
                const int t = u / CH;
                const int c = u - t * CH;
                const size_t src = (size_t)slot_pixel(gg, w.wy, w.wx, t) * D + c * EPC;
                *reinterpret_cast<uint4*>(dst + t * ROWB + ((c ^ kswz<CH>(t)) * 16)) =
                    *reinterpret_cast<const uint4*>(src_plane + src);
            }
        } else {
            stage_rows<T, D>(dst, KSTR, src_plane, gg, w.wy, w.wx);
        }
    };
    stage_k(Ks, Kh, g);
    if (DUAL) stage_k(Ks + N * KSTR, K1h, g1);
    __syncthreads();

    const int row0 = w.part * p.rows_per_block;
    const int row1 = min(N, row0 + p.rows_per_block);
    const int K_l = p.K_l;
    const float scale2 = p.scale2;

    // The batch's query rows (NK sets x 4 rows) pass through the wave's histogram
    // words: the next batch's are loaded after this batch's keys and written there
    // once the selection is done with them, before the I/A stores. Loaded after the
    // stores, they would wait for the stores too (one in-order vmcnt counter), and
    // with them the next batch's MFMAs (4 % faster on the fused bf16 kernel). With a
    // previous map (HAS_A) the two registers this holds across the selection made the
    // kernel spill, so there the rows are loaded at the MFMA phase.
    constexpr bool QLDS = !HAS_A;
    constexpr int QW = NK * 4 * ROWB / 4;   // words of a batch's query rows
    constexpr int NQ = (QW + kWave - 1) / kWave;
    static_assert(QW <= 4 * HISTG, "query rows exceed the wave's histogram words");
    unsigned* qst = hist0 + wave * 4 * HISTG;
    auto load_q = [&](int nb, unsigned (&qd)[NQ]) {
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const int u = lane + kWave * k;
            qd[k] = 0u;
            if (u < QW) {
                const int sr = u / (ROWB / 4);   // set * 4 + row
                const int st = sr >> 2, r = sr & 3;
                const bool f = DUAL && st == 0;
                const int iq = min(nb + r, row1 - 1);
                const unsigned* qr = reinterpret_cast<const unsigned*>((f ? Q1h : Qh) +
                                                                       (size_t)slot_pixel(f ? g1 : g, w.wy, w.wx, iq) * D);
                qd[k] = qr[u - sr * (ROWB / 4)];
            }
        }
    };
    auto put_q = [&](const unsigned (&qd)[NQ]) {
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const int u = lane + kWave * k;
            if (u < QW) qst[u] = qd[k];
        }
    };
    if constexpr (QLDS) {
        unsigned q0[NQ];
        load_q(row0 + wave * 4, q0);
        put_q(q0);
    }
    for (int base = row0 + wave * 4; base < row1; base += NW * 4) {
        // per-lane values are re-derived every batch from the lane index, itself
        // recomputed by v_mbcnt in an asm block the compiler cannot hoist: kept live
        // across the loop, the lane index, its group, the histogram addresses and
        // the KPT slot indices would not fit the register budget of 4 waves per SIMD
        // (they were spilled and reloaded at the top of every batch, behind the
        // previous batch's stores)
        int lv;
        __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lv));
        const int gv = lv >> 4;
        unsigned* hbv = hist0 + (wave * 4 + gv) * HISTG;
        const int glv = lv & (GL - 1);
        // 16 accumulator chains (one per 64-candidate tile), contraction chunk outer:
        // one 16-byte chunk of the query is live at a time
        // wave priority: the VALU-heavy selection of one wave issues ahead of the
        // MFMA phase of the others on its SIMD (measured 3-4 % faster than equal
        // priorities)
        __builtin_amdgcn_s_setprio(0);
        v4f acc[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int set = 0; set < NK; ++set) {   // DUAL: the first layer's q1.k1, then q.k
            const bool first = DUAL && set == 0;
            // each set's K offset derived here from an opaque copy of the lane index (kept
            // live from the top of the batch through the first set's MFMAs, it was spilled)
            int lvs = lv;
            __asm__ volatile("" : "+v"(lvs));
            // this lane's A-operand row (lv & 3) of the set: from the wave's LDS words, or
            // (HAS_A) from global memory
            const unsigned char* qrow =
                QLDS ? reinterpret_cast<const unsigned char*>(qst) + (set * 4 + (lvs & 3)) * ROWB
                     : reinterpret_cast<const unsigned char*>(
                           (first ? Q1h : Qh) +
                           (size_t)slot_pixel(first ? g1 : g, w.wy, w.wx, min(base + (lvs & 3), row1 - 1)) * D);
            const unsigned char* kr0 = Ks + (first ? N * KSTR : 0) + lvs * KSTR;
            uint4 qc[CH];
#pragma unroll
            for (int m = 0; m < CH; ++m) qc[m] = *reinterpret_cast<const uint4*>(qrow + 16 * m);
            // tiles in groups of TG (TG independent accumulator chains), contraction chunk
            // inner: at most TG x CH K chunks in flight. TG = 4 leaves the kernels without
            // spills (16 spilled up to 5 dwords; with the lane values above kept live, the
            // fused kernel spilled at every TG, and 7 dwords per batch at TG = 16)
            constexpr int TG = 4;
#pragma unroll
            for (int t0 = 0; t0 < 16; t0 += TG) {
#pragma unroll
                for (int m = 0; m < CH; ++m) {
                    const int koff = (SWZ ? (m ^ kswz<CH>(lv)) : m) * 16;
#pragma unroll
                    for (int t = t0; t < t0 + TG; ++t)
                        acc[t] = Mfma4<T>::chunk(qc[m], *reinterpret_cast<const uint4*>(kr0 + kWave * t * KSTR + koff),
                                                 acc[t]);
                }
            }
        }
        __builtin_amdgcn_s_setprio(2);
        // Selection in the MFMA output layout: acc[t][r] = s(row base + r, candidate
        // 64t + lane), so a row's 1024 keys lie in 16 registers across the whole wave,
        // in ascending candidate order over (t, lane). Per-row values (maximum, radix
        // interval, sums) are wave-uniform and sit in scalar registers; a row whose
        // threshold is found skips the remaining radix levels of the batch, and a kept
        // entry's position is one mbcnt over the row's ballot plus a scalar count.
        int lv2;
        __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lv2));
        unsigned* hw = hist0 + wave * 4 * HISTG;   // the wave's 4 row histograms
        float uv[4][16];                            // key of row r, candidate 64t + lane
        {
            // keys u = A^{l-1} exp2(scale2 (s - max s)); A^{l-1} is loaded now, two rows
            // at a time (16 waves per CU cover the load latency)
            float mx[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                mx[r] = acc[0][r];
#pragma unroll
                for (int t = 1; t < 16; ++t) mx[r] = fmaxf(mx[r], acc[t][r]);
            }
            const float cg = -rows4_to_groups(mx, MaxF()) * scale2;   // row lane >> 4
            float c[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) c[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cg), 16 * r));
            const float* abase = HAS_A ? p.A_prev + (size_t)w.wh * N * N + lv2 : nullptr;
#pragma unroll
            for (int h = 0; h < 4; h += 2) {
                float ab[2][16];
                if (HAS_A) {
#pragma unroll
                    for (int rr = 0; rr < 2; ++rr) {
                        const float* ar = abase + (size_t)min(base + h + rr, N - 1) * N;
#pragma unroll
                        for (int t = 0; t < 16; ++t) ab[rr][t] = ar[kWave * t];
                    }
                }
#pragma unroll
                for (int rr = 0; rr < 2; ++rr)
#pragma unroll
                    for (int t = 0; t < 16; ++t) {
                        const float e = fast_exp2(fmaf(acc[t][h + rr], scale2, c[h + rr]));
                        uv[h + rr][t] = HAS_A ? fmaxf(ab[rr][t] * e, 0.0f) : e;
                    }
                __asm__ volatile("" ::: "memory");   // the second pair's loads go out after the first is used
            }
        }

        // the next batch's query rows: loads in flight during the selection
        unsigned qn[NQ];
        const bool more = QLDS && base + NW * 4 < row1;
        if (more) load_q(base + NW * 4, qn);

        // Exact K_l-th largest key of each row by radix descent over the fp32 bit
        // patterns (u >= 0, so integer order is float order): the row's interval
        // [lo, hi) is cut into 128 bins of 2^shift keys counted with LDS atomics; the
        // 16 lanes of group g then scan row g's bins in descending order (8 per lane)
        // and publish the bin holding the need-th key; keys above it are kept, and the
        // search descends into it. A row ends when the bin's keys are all needed or all
        // equal: every key > tau = lo is kept, need more among the n_tau keys == tau.
        const unsigned act = (1u << max(0, min(4, row1 - base))) - 1u;   // rows below row1
        int lo[4], hi[4], need[4], ntau[4];
        unsigned done = ~act & 0xFu;
        {
            int mn[4], mk[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                mn[r] = 0x7fffffff;
                mk[r] = -1;
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    mn[r] = min(mn[r], __float_as_int(uv[r][t]));
                    mk[r] = max(mk[r], __float_as_int(uv[r][t]));
                }
            }
            const int mng = rows4_to_groups_i(mn, MinI());
            const int mkg = rows4_to_groups_i(mk, MaxI());
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                lo[r] = __builtin_amdgcn_readlane(mng, 16 * r);
                hi[r] = __builtin_amdgcn_readlane(mkg, 16 * r) + 1;
                need[r] = K_l;
                ntau[r] = 0;
                if ((act >> r & 1u) && hi[r] - lo[r] <= 1) {   // all keys equal
                    done |= 1u << r;
                    ntau[r] = N;
                }
            }
        }
        {
            const int g = lv2 >> 4;
            const int gl = lv2 & (GL - 1);
            unsigned* hg = hw + g * HISTG;   // the histogram this lane scans (row g)
            while (done != 0xFu) {
                int shift[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) shift[r] = max(32 - __clz(max(hi[r] - lo[r], 2) - 1) - 7, 0);
                {
                    // zeros made here (a zero quad kept live across the loop was spilled)
                    unsigned z;
                    __asm__ volatile("v_mov_b32 %0, 0" : "=v"(z));
                    *reinterpret_cast<uint4*>(hg + BPL * gl) = make_uint4(z, z, z, z);
                    *reinterpret_cast<uint4*>(hg + BPL * gl + 4) = make_uint4(z, z, z, z);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (done >> r & 1u) continue;
                    unsigned* hr = hw + r * HISTG;
                    const unsigned range = (unsigned)(hi[r] - lo[r]);
#pragma unroll
                    for (int t = 0; t < 16; ++t) {
                        const unsigned dk = (unsigned)(__float_as_int(uv[r][t]) - lo[r]);
                        if (dk < range) atomicAdd(&hr[dk >> shift[r]], 1u);
                    }
                }
                __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                // group g's lanes hold bins 127 - 8 gl - b, b = 0..7 (descending key order)
                const int needl = g == 0 ? need[0] : g == 1 ? need[1] : g == 2 ? need[2] : need[3];
                unsigned cb[BPL];
#pragma unroll
                for (int b = 0; b < BPL; b += 4) {
                    const uint4 c4 = *reinterpret_cast<const uint4*>(hg + HISTG - BPL * (gl + 1) + b);
                    cb[BPL - 1 - b] = c4.x;
                    cb[BPL - 2 - b] = c4.y;
                    cb[BPL - 3 - b] = c4.z;
                    cb[BPL - 4 - b] = c4.w;
                }
                unsigned lsum = 0;
#pragma unroll
                for (int b = 0; b < BPL; ++b) lsum += cb[b];
                unsigned run = Grp<GL>::incl_scan(lsum) - lsum;
                // exactly one bin of a searching row matches; its result goes to the row's
                // words 0..2 (their counts have been read by then). Rows already done
                // have empty histograms and match nothing.
#pragma unroll
                for (int b = 0; b < BPL; ++b) {
                    if (run < (unsigned)needl && run + cb[b] >= (unsigned)needl) {
                        hg[0] = (unsigned)(HISTG - 1 - BPL * gl - b);
                        hg[1] = run;
                        hg[2] = cb[b];
                    }
                    run += cb[b];
                }
                __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (done >> r & 1u) continue;
                    const unsigned* res = hw + r * HISTG;
                    const int bin = __builtin_amdgcn_readfirstlane((int)res[0]);
                    const int above = __builtin_amdgcn_readfirstlane((int)res[1]);
                    const int in_bin = __builtin_amdgcn_readfirstlane((int)res[2]);
                    need[r] -= above;
                    lo[r] += bin << shift[r];
                    hi[r] = min(hi[r], lo[r] + (1 << shift[r]));
                    if (in_bin == need[r] || hi[r] - lo[r] <= 1) {   // whole bin kept, or all its keys equal
                        ntau[r] = in_bin;
                        done |= 1u << r;
                    }
                }
                __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
        }

        // tau = lo, need_tau = need. A tie (more keys equal tau than needed) keeps the
        // lowest candidates among them, by rank in the store loop; thr = tau - 1 keeps
        // every key equal to tau, thr = tau (tie rows) adds them by rank.
        bool tie[4];
        int thr[4];
        bool any_tie = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            tie[r] = (act >> r & 1u) && ntau[r] > need[r];
            thr[r] = tie[r] ? lo[r] : lo[r] - 1;
            any_tie = any_tie || tie[r];
        }
        float inv[4];
        {
            float ks[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                ks[r] = 0.0f;
#pragma unroll
                for (int t = 0; t < 16; ++t) ks[r] += __float_as_int(uv[r][t]) > thr[r] ? uv[r][t] : 0.0f;
            }
            float ksg = rows4_to_groups(ks, SumF());   // row lane >> 4
            if (any_tie) {
                const int g = lv2 >> 4;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (tie[r] && g == r) ksg += (float)need[r] * __int_as_float(lo[r]);
            }
            const float invg = 1.0f / ksg;
#pragma unroll
            for (int r = 0; r < 4; ++r) inv[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(invg), 16 * r));
        }
        if (more) put_q(qn);   // the histogram words are free again

        // Stores: one buffer store of I and of A per register and row; entries not
        // kept get an offset past the resource's range, which the hardware drops.
        // Rows past row1 (last batch) are not stored.
        const size_t rbase = ((size_t)w.wh * N + base) * K_l;
        const int nbytes = max(0, min(4, row1 - base)) * K_l * 4;
        const __amdgpu_buffer_rsrc_t rI = make_rsrc(p.I_out + rbase, nbytes);
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A_out + rbase, nbytes);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (!(act >> r & 1u)) continue;
            // copies the compiler cannot see through, so the comparisons are not kept
            // alive as lane masks from the sums above
            int thr2 = thr[r], tau2 = lo[r];
            __asm__ volatile("" : "+s"(thr2), "+s"(tau2));
            const int roff = r * K_l;
            const float ir = inv[r];
            int ob = 0;   // entries of the row stored so far
            auto emit = [&](int t, bool k) {
                const uint64_t m = ballot(k);
                // pos is made opaque so that the offset stays a select, not a branch
                int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)ob));
                __asm__ volatile("" : "+v"(pos));
                const int off = k ? (roff + pos) * 4 : 0x7FFFFFF0;
                __builtin_amdgcn_raw_buffer_store_b32(kWave * t + lv2, rI, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(uv[r][t] * ir), rA, off, 0, 0);
                ob += popc(m);
            };
            if (!tie[r]) {
#pragma unroll
                for (int t = 0; t < 16; ++t) emit(t, __float_as_int(uv[r][t]) > thr2);
            } else {
                int tb = 0;   // keys equal to tau met so far in the row
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const bool eq = __float_as_int(uv[r][t]) == tau2;
                    const uint64_t me = ballot(eq);
                    const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(me >> 32),
                                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)me, (uint32_t)tb));
                    tb += popc(me);
                    emit(t, __float_as_int(uv[r][t]) > thr2 || (eq && rank < need[r]));
                }
            }
        }
    }
}

// O_i = sum_j A^l_ij v_j from stored (I^l, A^l) rows, V of the window in LDS: the
// second half of a layer whose K and V do not fit in LDS together.
template <typename T, int D, int GL, int NW>
__global__ __launch_bounds__(NW * kWave) void aggregate_kernel(const SparseArgs p) {
    constexpr int EPC = Chunk<T>::kElems;
    constexpr int CH = D / EPC;
    constexpr int ROWB = D * (int)sizeof(T);
    constexpr int RPW = kWave / GL;
    constexpr int GS = GL / CH;   // entries in flight per row
    extern __shared__ __align__(16) unsigned char smem[];

    const Geom g = p.g;
    const int N = g.N;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int grp = lane / GL;
    const int gl = lane & (GL - 1);
    const int vchunk = gl % CH;
    const int vsub = gl / CH;
    const WhPart w = decode_block(p.blocks_per_wh, p.xcd_map, g);
    const size_t plane = (size_t)w.bh * g.H * g.W * D;
    const T* Vh = static_cast<const T*>(p.V) + plane;
    float* Oh = p.O_out + plane;
    stage_rows<T, D>(smem, ROWB, Vh, g, w.wy, w.wx);
    __syncthreads();

    const int row0 = w.part * p.rows_per_block;
    const int row1 = min(N, row0 + p.rows_per_block);
    const int K_l = p.K_l;
    for (int base = row0 + wave * RPW; base < row1; base += NW * RPW) {
        const int i_raw = base + grp;
        const bool active = i_raw < row1;
        const int i = active ? i_raw : row0;
        const size_t row = (size_t)w.wh * N + i;
        const int32_t* Ir = p.I_out + row * K_l;
        const float* Ar = p.A_out + row * K_l;
        float oacc[EPC];
#pragma unroll
        for (int x = 0; x < EPC; ++x) oacc[x] = 0.0f;
        const int cnt = active ? K_l : 0;
        for (int e0 = vsub * 4; e0 < cnt; e0 += 4 * GS) {
            int jv[4];
            float wv[4];
            if ((K_l & 3) == 0 && e0 + 4 <= cnt) {   // 16-byte aligned rows
                const int4 j4 = *reinterpret_cast<const int4*>(Ir + e0);
                const float4 w4 = *reinterpret_cast<const float4*>(Ar + e0);
                jv[0] = j4.x; jv[1] = j4.y; jv[2] = j4.z; jv[3] = j4.w;
                wv[0] = w4.x; wv[1] = w4.y; wv[2] = w4.z; wv[3] = w4.w;
            } else {
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    jv[x] = e0 + x < cnt ? Ir[e0 + x] : 0;
                    wv[x] = e0 + x < cnt ? Ar[e0 + x] : 0.0f;
                }
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                if (e0 + x >= cnt) break;   // padding past K_l: no term (0 * a non-finite V would be NaN)
                const int j = (int)min((unsigned)jv[x], (unsigned)(N - 1));
                float vf[EPC];
                Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(smem + j * ROWB + vchunk * 16), vf);
#pragma unroll
                for (int y = 0; y < EPC; ++y) oacc[y] = fmaf(wv[x], vf[y], oacc[y]);
            }
        }
#pragma unroll
        for (int x = 0; x < EPC; ++x) oacc[x] = reduce_chunk_lanes<CH, GL>(oacc[x]);
        if (active && vsub == 0) {
            float* orow = Oh + (size_t)slot_pixel(g, w.wy, w.wx, i) * D + vchunk * EPC;
#pragma unroll
            for (int x = 0; x < EPC; x += 4)
                *reinterpret_cast<float4*>(orow + x) = make_float4(oacc[x], oacc[x + 1], oacc[x + 2], oacc[x + 3]);
        }
    }
}

// Same result for K_l <= 256 and K_l % 4 == 0, organised for memory-level
// parallelism: a wavefront takes R consecutive query rows per step, whose I^l /
// A^l entries are one contiguous run of R*K_l <= 256 entries, loaded with one
// 16-byte load per lane for I and one for A, a step ahead of their use. The
// entries are staged in a per-wave LDS buffer; a group of GL = 64/R lanes then
// accumulates one row, CH lanes per V row (one 16-byte chunk each), GS = GL/CH
// entries of the row at a time, 4 consecutive entries per LDS read.
template <typename T, int D, int R, int NW>
__global__ __launch_bounds__(NW * kWave) void aggregate_rows_kernel(const SparseArgs p) {
    constexpr int EPC = Chunk<T>::kElems;
    constexpr int CH = D / EPC;
    constexpr int ROWB = D * (int)sizeof(T);
    constexpr int GL = kWave / R;
    constexpr int GS = GL / CH;
    static_assert(GS >= 1, "a row needs at least CH lanes");
    extern __shared__ __align__(16) unsigned char smem[];

    const Geom g = p.g;
    const int N = g.N;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int grp = lane / GL;
    const int gl = lane & (GL - 1);
    const int vchunk = gl % CH;
    const int vsub = gl / CH;
    const WhPart w = decode_block(p.blocks_per_wh, p.xcd_map, g);
    const size_t plane = (size_t)w.bh * g.H * g.W * D;
    const T* Vh = static_cast<const T*>(p.V) + plane;
    float* Oh = p.O_out + plane;
    int* sj = reinterpret_cast<int*>(smem + N * ROWB) + wave * 512;   // 256 V-row offsets, then 256 weights
    float* sw = reinterpret_cast<float*>(sj + 256);
    const int K_l = p.K_l;
    const int row0 = w.part * p.rows_per_block;
    const int row1 = min(N, row0 + p.rows_per_block);
    const int32_t* Iw = p.I_out + (size_t)w.wh * N * K_l;
    const float* Aw = p.A_out + (size_t)w.wh * N * K_l;
    int4 jn = make_int4(0, 0, 0, 0);
    float4 wn = make_float4(0.f, 0.f, 0.f, 0.f);
    auto load = [&](int base) {   // entries [base*K_l, min(base+R, row1)*K_l) of the window-head
        const int e = base * K_l + lane * 4;
        if (e < min(base + R, row1) * K_l) {
            jn = *reinterpret_cast<const int4*>(Iw + e);
            wn = *reinterpret_cast<const float4*>(Aw + e);
        }
    };
    int base = row0 + wave * R;
    if (base < row1) load(base);   // before the staging: the latency overlaps it
    stage_rows<T, D>(smem, ROWB, Vh, g, w.wy, w.wx);
    __syncthreads();
    const unsigned char* vbase = smem + vchunk * 16;   // this lane's 16-byte chunk of every V row
    for (; base < row1; base += NW * R) {
        // stage byte offsets of the V rows (slot clamped to the window: memory safety only)
        const unsigned nm = (unsigned)(N - 1);
        const int4 off = make_int4((int)min((unsigned)jn.x, nm) * ROWB, (int)min((unsigned)jn.y, nm) * ROWB,
                                   (int)min((unsigned)jn.z, nm) * ROWB, (int)min((unsigned)jn.w, nm) * ROWB);
        *reinterpret_cast<int4*>(sj + lane * 4) = off;
        *reinterpret_cast<float4*>(sw + lane * 4) = wn;
        if (base + NW * R < row1) load(base + NW * R);
        const int i = base + grp;
        float oacc[EPC];
#pragma unroll
        for (int x = 0; x < EPC; ++x) oacc[x] = 0.0f;
        if (i < row1) {
            const int* rj = sj + grp * K_l;
            const float* rw = sw + grp * K_l;
            for (int e = vsub * 4; e < K_l; e += GS * 4) {
                const int4 o4 = *reinterpret_cast<const int4*>(rj + e);
                const float4 w4 = *reinterpret_cast<const float4*>(rw + e);
                const int ov[4] = {o4.x, o4.y, o4.z, o4.w};
                const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
                float vf[4][EPC];
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(vbase + ov[x]), vf[x]);
#pragma unroll
                for (int x = 0; x < 4; ++x)
#pragma unroll
                    for (int y = 0; y < EPC; ++y) oacc[y] = fmaf(wv[x], vf[x][y], oacc[y]);
            }
        }
#pragma unroll
        for (int x = 0; x < EPC; ++x) oacc[x] = reduce_chunk_lanes<CH, GL>(oacc[x]);
        if (i < row1 && vsub == 0) {
            float* orow = Oh + (size_t)slot_pixel(g, w.wy, w.wx, i) * D + vchunk * EPC;
#pragma unroll
            for (int x = 0; x < EPC; x += 4)
                *reinterpret_cast<float4*>(orow + x) = make_float4(oacc[x], oacc[x + 1], oacc[x + 2], oacc[x + 3]);
        }
    }
}


// 4-chunk V rows (bf16 d = 32, fp32 d = 16): one lane quad per row group, one
// 16-byte chunk per lane. A row takes GL = 64 / R lanes (GL / 4 quads); its entries
// are handed out in S rounds of 4 steps: at round r, lane c of quad q loads step c
// (4 consecutive (I, A) pairs at 4 GL r + GL c + 4 q; the wave's loads cover whole
// row segments, coalesced), and at step k the quad takes lane k's entries by a DPP
// quad broadcast, so LDS carries only V rows. With more rounds a row needs fewer
// quads, and the closing sum over the row's quads (two cross-lane exchanges and an
// add per quad halving, 8 values) is paid once per 16 S entries per quad instead
// of per 16 (layer 2: 4 quads of 64 entries instead of 16 of 16).
template <typename T, int D, int R, int NW, int S>
__global__ __launch_bounds__(NW * kWave) void aggregate_quads_kernel(const SparseArgs p) {
    constexpr int EPC = Chunk<T>::kElems;
    constexpr int ROWB = D * (int)sizeof(T);
    constexpr int GL = kWave / R;   // lanes per row
    static_assert(D / EPC == 4, "one 16-byte chunk per lane of a quad");
    static_assert(GL >= 4, "a row needs a quad");
    extern __shared__ __align__(16) unsigned char smem[];

    const Geom g = p.g;
    const int N = g.N;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int grp = lane / GL;
    const int gl = lane & (GL - 1);
    const int q = gl >> 2;
    const int c = gl & 3;
    const WhPart w = decode_block(p.blocks_per_wh, p.xcd_map, g);
    const size_t plane = (size_t)w.bh * g.H * g.W * D;
    const T* Vh = static_cast<const T*>(p.V) + plane;
    float* Oh = p.O_out + plane;

    const int K_l = p.K_l;   // a multiple of 4, at most 4 GL S
    const int row0 = w.part * p.rows_per_block;
    const int row1 = min(N, row0 + p.rows_per_block);
    // the window-head's (I, A) rows through buffer resources: a load past the rows'
    // range returns zeros (no branch around the loads)
    const int wh_bytes = N * K_l * 4;
    const __amdgpu_buffer_rsrc_t rI = make_rsrc(p.I_out + (size_t)w.wh * N * K_l, wh_bytes);
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A_out + (size_t)w.wh * N * K_l, wh_bytes);
    const int e0 = GL * c + 4 * q;   // this lane's entries at round r: e0 + 4 GL r
    // round r of the rows at b: offsets past the range for inactive rows and entries past K_l
    auto load_round = [&](int b, int r, int4& jv, float4& wv) {
        const int i = b + grp;
        const int e = e0 + 4 * GL * r;
        const int off = (i < row1 && e < K_l) ? (i * K_l + e) * 4 : 0x7FFFFFF0;
        const auto jr = __builtin_amdgcn_raw_buffer_load_b128(rI, off, 0, 0);
        const auto wr = __builtin_amdgcn_raw_buffer_load_b128(rA, off, 0, 0);
        jv = make_int4((int)jr[0], (int)jr[1], (int)jr[2], (int)jr[3]);
        wv = make_float4(__uint_as_float(wr[0]), __uint_as_float(wr[1]), __uint_as_float(wr[2]),
                         __uint_as_float(wr[3]));
    };
    // the next round's entries are loaded one round ahead (the first before the staging)
    int4 jn;
    float4 wn;
    load_round(row0 + wave * R, 0, jn, wn);
    stage_rows<T, D>(smem, ROWB, Vh, g, w.wy, w.wx);
    __syncthreads();

    for (int base = row0 + wave * R; base < row1; base += NW * R) {
        const int i = base + grp;
        const bool active = i < row1;
        float acc[EPC];
#pragma unroll
        for (int y = 0; y < EPC; ++y) acc[y] = 0.0f;
#pragma unroll
        for (int r = 0; r < S; ++r) {
            const int4 jm = jn;
            const float4 wm = wn;
            if (r + 1 < S) load_round(base, r + 1, jn, wn);
            else if (base + NW * R < row1) load_round(base + NW * R, 0, jn, wn);
            auto step = [&](auto kc) {
                constexpr int KC = decltype(kc)::value;
                constexpr int BC = KC * 0x55;   // quad_perm [k, k, k, k]
                const int jk[4] = {dpp<BC>(jm.x), dpp<BC>(jm.y), dpp<BC>(jm.z), dpp<BC>(jm.w)};
                const float wk[4] = {dppf<BC>(wm.x), dppf<BC>(wm.y), dppf<BC>(wm.z), dppf<BC>(wm.w)};
                // quads whose step-k entries lie past K_l add nothing: 0 * a non-finite V
                // row would turn O into NaN
                if (4 * GL * r + GL * KC + 4 * q >= K_l) return;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int j = (int)min((unsigned)jk[x], (unsigned)(N - 1));   // memory safety only
                    float vf[EPC];
                    Chunk<T>::to_f32(*reinterpret_cast<const uint4*>(smem + j * ROWB + c * 16), vf);
#pragma unroll
                    for (int y = 0; y < EPC; ++y) acc[y] = fmaf(wk[x], vf[y], acc[y]);
                }
            };
            if (4 * GL * r < K_l) {   // uniform: the round holds entries
                step(std::integral_constant<int, 0>());
                if (4 * GL * r + GL < K_l) step(std::integral_constant<int, 1>());
                if (4 * GL * r + 2 * GL < K_l) step(std::integral_constant<int, 2>());
                if (4 * GL * r + 3 * GL < K_l) step(std::integral_constant<int, 3>());
            }
        }
#pragma unroll
        for (int y = 0; y < EPC; ++y) acc[y] = reduce_chunk_lanes<4, GL>(acc[y]);   // the row's quads
        if (active && q == 0) {
            float* orow = Oh + (size_t)slot_pixel(g, w.wy, w.wx, i) * D + c * EPC;
#pragma unroll
            for (int y = 0; y < EPC; y += 4)
                *reinterpret_cast<float4*>(orow + y) = make_float4(acc[y], acc[y + 1], acc[y + 2], acc[y + 3]);
        }
    }
}

template <class F>
hipError_t launch_fn(F fn, const SparseArgs& a, int threads, int lds, int grid, hipStream_t s) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(threads), lds, s, a);
    return hipGetLastError();
}

template <typename T, int D, int GL, int KPT, int MODE>
hipError_t launch_one(const SparseArgs& a, int lds, int grid, hipStream_t s) {
    constexpr int NW = (KPT <= 4 || (MODE == kKselect && (KPT <= 8 || (KPT <= 16 && sizeof(T) == 2)))) ? 16 : 8;
    constexpr bool PQ = KPT <= 4 && D * sizeof(T) <= 64;   // prefetch q when registers allow
    if constexpr (MODE == kKselect) {
        if (a.bias) {
            if (a.K_prev == GL * KPT)
                return launch_fn(sparse_layer_kernel<T, D, GL, KPT, MODE, NW, PQ, true, true>, a, NW * kWave, lds,
                                 grid, s);
            return launch_fn(sparse_layer_kernel<T, D, GL, KPT, MODE, NW, PQ, false, true>, a, NW * kWave, lds, grid,
                             s);
        }
    }
    if (MODE == kKselect && a.K_prev == GL * KPT)
        return launch_fn(sparse_layer_kernel<T, D, GL, KPT, MODE, NW, PQ, true>, a, NW * kWave, lds, grid, s);
    return launch_fn(sparse_layer_kernel<T, D, GL, KPT, MODE, NW, PQ, false>, a, NW * kWave, lds, grid, s);
}

template <typename T, int D, int GL, int KPT>
hipError_t launch_mode(const SparseArgs& a, SparseMode mode, int lds, int grid, hipStream_t s) {
    switch (mode) {
        case kKselect: return launch_one<T, D, GL, KPT, kKselect>(a, lds, grid, s);
        default: return launch_one<T, D, GL, KPT, kKVglobal>(a, lds, grid, s);
    }
}

template <typename T, int D>
hipError_t launch_shape(const SparseArgs& a, SparseMode mode, int lds, int grid, hipStream_t s) {
    const int kp = a.K_prev;
    if (mode == kKselect && kp <= 256) {
        // selection only: narrow row groups (4 to 16 lanes, 16 to 4 rows per wavefront)
        // amortise the per-row reductions and scans over more candidates per lane
        // (4-lane groups for K_prev <= 32 and 8-lane groups for K_prev <= 64 measured
        // 30 % and 11 % faster than 16-lane groups on the bf16 640x384 chain)
        if (kp <= 16) return launch_one<T, D, 4, 4, kKselect>(a, lds, grid, s);
        if (kp <= 32) return launch_one<T, D, 4, 8, kKselect>(a, lds, grid, s);
        if (kp <= 64) return launch_one<T, D, 8, 8, kKselect>(a, lds, grid, s);
        if (kp <= 128) return launch_one<T, D, 16, 8, kKselect>(a, lds, grid, s);
        // K_prev <= 256: bf16 takes 4 rows of 16 candidates per lane per wavefront
        // (more independent gathers in flight per wave); fp32 2 rows of 8 (16 would not
        // fit the 128 VGPRs of 16-wave workgroups)
        if constexpr (sizeof(T) == 2) return launch_one<T, D, 16, 16, kKselect>(a, lds, grid, s);
        return launch_one<T, D, 32, 8, kKselect>(a, lds, grid, s);
    }
    if (kp <= 16) return launch_mode<T, D, 16, 1>(a, mode, lds, grid, s);
    if (kp <= 32) return launch_mode<T, D, 16, 2>(a, mode, lds, grid, s);
    if (kp <= 64) return launch_mode<T, D, 16, 4>(a, mode, lds, grid, s);
    if (kp <= 128) return launch_mode<T, D, 32, 4>(a, mode, lds, grid, s);
    if (kp <= 256) return launch_mode<T, D, 64, 4>(a, mode, lds, grid, s);
    if (kp <= 512) return launch_mode<T, D, 64, 8>(a, mode, lds, grid, s);
    return launch_mode<T, D, 64, 16>(a, mode, lds, grid, s);
}

template <typename T, int D>
constexpr int all_cand_kstr() {
    constexpr int ROWB = D * (int)sizeof(T);
    return (ROWB == 128 || ROWB == 64) ? ROWB : ROWB + 16;
}
constexpr int kAllCandHistBytes = 16 * 4 * (8 * 16) * 4;   // 16 waves x 4 rows x 128 bins

template <typename T, int D>
hipError_t launch_all_cand_t(const SparseArgs& a, int grid, hipStream_t s) {
    const int lds = 1024 * all_cand_kstr<T, D>() + kAllCandHistBytes;
    if (a.A_prev) return launch_fn(all_cand_rows_kernel<T, D, true, false>, a, 16 * kWave, lds, grid, s);
    return launch_fn(all_cand_rows_kernel<T, D, false, false>, a, 16 * kWave, lds, grid, s);
}

template <typename T, int D>
hipError_t launch_all_cand_dual_t(const SparseArgs& a, int grid, hipStream_t s) {
    if constexpr (2 * 1024 * all_cand_kstr<T, D>() + kAllCandHistBytes > kLdsBytes) {
        return hipErrorInvalidValue;   // rejected by the caller beforehand
    } else {
        const int lds = 2 * 1024 * all_cand_kstr<T, D>() + kAllCandHistBytes;
        return launch_fn(all_cand_rows_kernel<T, D, false, true>, a, 16 * kWave, lds, grid, s);
    }
}

template <typename T, int D>
hipError_t launch_aggregate_t(const SparseArgs& a, int grid, hipStream_t s) {
    const int lds = a.g.N * D * (int)sizeof(T);
    // 4-chunk V rows: entries broadcast within quads (4-17 % faster on the bf16 patch
    // batch); with 8 chunks, two per lane of a quad, that was measured slower than
    // staging the entries in LDS for 8-lane rows (0.33 against 0.30 ms at layer 2)
    if constexpr (D / Chunk<T>::kElems == 4) {
        if (a.K_l <= 256 && a.K_l % 4 == 0 && lds <= kLdsBytes) {
            // up to 64 entries per quad (4 rounds): GL = max(4, K_l / 16) lanes per row
            const int kl = a.K_l;
            if (kl <= 16) return launch_fn(aggregate_quads_kernel<T, D, 16, 16, 1>, a, 16 * kWave, lds, grid, s);
            if (kl <= 32) return launch_fn(aggregate_quads_kernel<T, D, 16, 16, 2>, a, 16 * kWave, lds, grid, s);
            if (kl <= 64) return launch_fn(aggregate_quads_kernel<T, D, 16, 16, 4>, a, 16 * kWave, lds, grid, s);
            if (kl <= 128) return launch_fn(aggregate_quads_kernel<T, D, 8, 16, 4>, a, 16 * kWave, lds, grid, s);
            return launch_fn(aggregate_quads_kernel<T, D, 4, 16, 4>, a, 16 * kWave, lds, grid, s);
        }
    }
    constexpr int RMAX = kWave / (D / Chunk<T>::kElems);   // rows per step with CH lanes per row
    if (a.K_l <= 256 && a.K_l % 4 == 0 && lds + 16 * 2048 <= kLdsBytes) {
        const int l2 = lds + 16 * 2048;
        const int r = 256 / a.K_l;   // rows whose entries fill one 16-byte load per lane
        if (r >= 16 && RMAX >= 16) return launch_fn(aggregate_rows_kernel<T, D, (RMAX >= 16 ? 16 : 1), 16>, a,
                                                    16 * kWave, l2, grid, s);
        if (r >= 8 && RMAX >= 8) return launch_fn(aggregate_rows_kernel<T, D, 8, 16>, a, 16 * kWave, l2, grid, s);
        if (r >= 4) return launch_fn(aggregate_rows_kernel<T, D, 4, 16>, a, 16 * kWave, l2, grid, s);
        if (r >= 2) return launch_fn(aggregate_rows_kernel<T, D, 2, 16>, a, 16 * kWave, l2, grid, s);
        return launch_fn(aggregate_rows_kernel<T, D, 1, 16>, a, 16 * kWave, l2, grid, s);
    }
    if (a.K_l <= 16) return launch_fn(aggregate_kernel<T, D, 16, 16>, a, 16 * kWave, lds, grid, s);
    if (a.K_l <= 32) return launch_fn(aggregate_kernel<T, D, 32, 16>, a, 16 * kWave, lds, grid, s);
    return launch_fn(aggregate_kernel<T, D, 64, 16>, a, 16 * kWave, lds, grid, s);
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

bool all_cand_dual_fits(int dtype, int D) {
    const int kstr = dtype == 0 ? (D == 16 ? all_cand_kstr<float, 16>() : all_cand_kstr<float, 32>())
                                : (D == 16 ? all_cand_kstr<uint16_t, 16>() : all_cand_kstr<uint16_t, 32>());
    return 2 * 1024 * kstr + kAllCandHistBytes <= kLdsBytes;
}

hipError_t launch_all_cand_dual(const SparseArgs& a, int dtype, int D, int grid, hipStream_t stream) {
    if (dtype == 0)
        return D == 16 ? launch_all_cand_dual_t<float, 16>(a, grid, stream)
                       : launch_all_cand_dual_t<float, 32>(a, grid, stream);
    return D == 16 ? launch_all_cand_dual_t<uint16_t, 16>(a, grid, stream)
                   : launch_all_cand_dual_t<uint16_t, 32>(a, grid, stream);
}

hipError_t launch_all_cand(const SparseArgs& a, int dtype, int D, int grid, hipStream_t stream) {
    if (dtype == 0)
        return D == 16 ? launch_all_cand_t<float, 16>(a, grid, stream)
                       : launch_all_cand_t<float, 32>(a, grid, stream);
    return D == 16 ? launch_all_cand_t<uint16_t, 16>(a, grid, stream)
                   : launch_all_cand_t<uint16_t, 32>(a, grid, stream);
}

hipError_t launch_aggregate(const SparseArgs& a, int dtype, int D, int grid, hipStream_t stream) {
    if (dtype == 0)
        return D == 16 ? launch_aggregate_t<float, 16>(a, grid, stream) : launch_aggregate_t<float, 32>(a, grid, stream);
    return D == 16 ? launch_aggregate_t<uint16_t, 16>(a, grid, stream)
                   : launch_aggregate_t<uint16_t, 32>(a, grid, stream);
}

}  // namespace pfa
