// C ABI of libpfa.so: argument validation, launch geometry, error mapping.
// The calls and their contracts are documented in include/pfa.h.
#include <math.h>

#include <mutex>
#include <vector>

#include "pfa.h"
#include "pfa_kernels.h"

namespace {

using pfa::Geom;

// Kernel timing: when enabled, each launch below is bracketed by two events
// recorded on its own stream. Records beyond the capacity are counted, not kept.
struct Timing {
    bool on = false;
    std::vector<hipEvent_t> ev;   // 2 per record
    std::vector<int32_t> kind;
    int32_t n = 0;
    int32_t dropped = 0;
};
Timing g_timing;

template <class F>
hipError_t timed(int32_t kind, hipStream_t s, F&& launch) {
    Timing& t = g_timing;
    if (!t.on) return launch();
    if (t.n >= (int32_t)t.kind.size()) {
        ++t.dropped;
        return launch();
    }
    hipError_t e = hipEventRecord(t.ev[2 * t.n], s);
    if (e != hipSuccess) return e;
    e = launch();
    if (e != hipSuccess) return e;
    e = hipEventRecord(t.ev[2 * t.n + 1], s);
    if (e != hipSuccess) return e;
    t.kind[t.n++] = kind;
    return hipSuccess;
}

void timing_release() {
    for (hipEvent_t e : g_timing.ev) (void)hipEventDestroy(e);
    g_timing = Timing();
}

constexpr int kVersion = 10000;  // 1.0.0

bool geom_from_shape(const pfa_shape* s, Geom* g, int* code) {
    *code = PFA_ERR_INVALID;
    if (!s) return false;
    if (s->B < 1 || s->heads < 1 || s->H < 1 || s->W < 1 || s->d < 1) return false;
    if (s->dtype != PFA_F32 && s->dtype != PFA_BF16) {
        *code = PFA_ERR_UNSUPPORTED;
        return false;
    }
    if (s->d != 16 && s->d != 32) {
        *code = PFA_ERR_UNSUPPORTED;
        return false;
    }
    if (s->win < 0) return false;
    g->B = s->B; g->heads = s->heads; g->H = s->H; g->W = s->W; g->d = s->d;
    g->win = s->win; g->shift = s->shift;
    if (s->win > 0) {
        if (s->H % s->win || s->W % s->win) return false;
        if (s->shift < 0 || s->shift >= s->win) return false;
        if (s->win > 32) {
            *code = PFA_ERR_UNSUPPORTED;
            return false;
        }
        g->N = s->win * s->win;
        g->nwy = s->H / s->win;
        g->nwx = s->W / s->win;
        g->win_magic = (65536 + s->win - 1) / s->win;
    } else {
        if (s->shift != 0) return false;
        if ((int64_t)s->H * s->W >= (1 << 24)) {
            *code = PFA_ERR_UNSUPPORTED;
            return false;
        }
        g->N = s->H * s->W;
        g->nwy = g->nwx = 1;
        g->win_magic = 0;
    }
    *code = PFA_OK;
    return true;
}

int elem_bytes(int dtype) { return dtype == PFA_F32 ? 4 : 2; }

// compute units of the current device (0 if the query fails: no split workloads)
int compute_units() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return cus;
}

int64_t n_wh(const Geom& g) { return (int64_t)g.B * g.heads * g.nwy * g.nwx; }

int run_sparse(const Geom& g, int dtype, const void* Q, const void* K, const void* V, const float* bias,
               const int32_t* I_prev, int i_shared, const float* A_prev, int K_prev, int K_l,
               int32_t* I_out, float* A_out, float* O_out, hipStream_t stream) {
    pfa::SparseArgs a;
    a.Q = Q; a.K = K; a.V = V;
    a.I_prev = I_prev; a.A_prev = A_prev;
    a.I_out = I_out; a.A_out = A_out; a.O_out = O_out;
    a.g = g;
    a.K_prev = K_prev; a.K_l = K_l;
    a.i_shared = i_shared ? 1 : 0;
    a.scale2 = (float)(1.4426950408889634 / sqrt((double)g.d));
    a.Q1 = nullptr; a.K1 = nullptr; a.shift1 = 0;
    a.bias = bias;

    const int rowb = g.d * elem_bytes(dtype);
    a.xcd_map = (n_wh(g) % 8 == 0) ? 1 : 0;
    if (g.win == 0) {
        a.blocks_per_wh = (g.N + 63) / 64;
        a.rows_per_block = 64;
        const int64_t grid = n_wh(g) * a.blocks_per_wh;
        if (grid > 0x7fffffff) return PFA_ERR_UNSUPPORTED;
        const hipError_t e = timed(PFA_KERNEL_SPARSE, stream, [&] {
            return pfa::launch_sparse(a, dtype, g.d, pfa::kKVglobal, pfa::kScratchBytes, (int)grid, stream);
        });
        return e == hipSuccess ? PFA_OK : PFA_ERR_HIP;
    }
    // two workgroups per window-head where the rows carry many candidates, or where
    // the window-heads are too few to fill the CUs four times over; otherwise one
    // (K_prev <= 128 on the 640x384 map: 2-4 % faster selections, the window's K
    // staged once per window-head instead of twice; on 384 window-heads one
    // workgroup each left CUs idle: the 256x256 map's layer-4 aggregation 0.10 ->
    // 0.12 ms)
    a.blocks_per_wh = (g.N >= 512 && (K_prev > 128 || n_wh(g) < 4 * (int64_t)compute_units())) ? 2 : 1;
    a.rows_per_block = (g.N + a.blocks_per_wh - 1) / a.blocks_per_wh;
    const int64_t grid64 = n_wh(g) * a.blocks_per_wh;
    if (grid64 > 0x7fffffff) return PFA_ERR_UNSUPPORTED;
    const int grid = (int)grid64;
    // Window mode: a selection kernel writes I^l / A^l (K of the window staged in
    // LDS), then the aggregation kernel forms O with V staged in LDS. Measured
    // faster than one kernel doing both, also where K and V fit in LDS together
    // (bf16): each kernel then runs with more waves and the selection with more
    // radix bins.
    hipError_t e;
    if (!I_prev && K_prev == 1024 && g.N == 1024 && !bias) {
        // every slot is a candidate: MFMA scores (with a bias, the gather kernel)
        e = timed(PFA_KERNEL_ALL_CANDIDATES, stream, [&] { return pfa::launch_all_cand(a, dtype, g.d, grid, stream); });
    } else {
        e = timed(PFA_KERNEL_SELECT, stream, [&] {
            return pfa::launch_sparse(a, dtype, g.d, pfa::kKselect, g.N * rowb + pfa::kScratchBytes, grid, stream);
        });
    }
    if (e == hipSuccess)
        e = timed(PFA_KERNEL_AGGREGATE, stream, [&] { return pfa::launch_aggregate(a, dtype, g.d, grid, stream); });
    return e == hipSuccess ? PFA_OK : PFA_ERR_HIP;
}

int run_dense_backward(const Geom& g, int dtype, const void* Q, const void* K, const void* V, const float* bias,
                       const float* lse, const float* dO, const float* dA, float* dQ, float* dK, float* dV,
                       float* Dws, hipStream_t s, float* dbias_rows = nullptr);
int run_sparse_backward(const pfa_shape* shape, const void* Q, const void* K, const void* V, const float* bias,
                        const int32_t* I_prev, const float* A_prev, int32_t K_prev, int32_t K_l, const int32_t* I_l,
                        const float* A_l, const float* dO, const float* dA_l, float* dQ, float* dK, float* dV,
                        float* dA_prev, float* dbias, void* workspace, int64_t workspace_bytes, hipStream_t s);

// workspace bytes: the sparse backward's g per kept pair and flag per row
int64_t sparse_bwd_ws(const Geom& g, int K_l) { return n_wh(g) * g.N * ((int64_t)K_l + 1) * 4; }
// per window-head bias-gradient tables
int64_t dbias_part_ws(const Geom& g) {
    const int64_t wrow = 2 * (int64_t)g.win - 1;
    return n_wh(g) * wrow * wrow * 4;
}
// the dense dQ kernel's per-wave rows of diagonal sums: [wh, N / 16, win, 64]
int64_t dense_dbias_rows_ws(const Geom& g) { return n_wh(g) * (g.N / 16) * (int64_t)g.win * 64 * 4; }
// backward of the fused first two layers: A^1 and dA^1 at the kept slots ([wh, N, K2]
// each), the dense dA^1 ([wh, N, N]), the sparse backward's workspace, the dense
// backward's (one fp32 per row)
int64_t fused_bwd_ws(const Geom& g, int K2) {
    return 2 * n_wh(g) * g.N * (int64_t)K2 * 4 + n_wh(g) * g.N * (int64_t)g.N * 4 + sparse_bwd_ws(g, K2) +
           n_wh(g) * g.N * 4;
}

}  // namespace

// Scratch memory of the no-allocation entry point (pfa_dense_layer_backward_noalloc):
// a static array in this file's device code object, so each GPU the library runs on
// holds its own copy, from the code object's load until the process ends. Host code
// never uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device (static_scratch below).
static __device__ __align__(256) unsigned char scratch[PFA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up on the first
// call on that device (with the device current) and kept.
int static_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return PFA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return PFA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PFA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PFA_OK;
}

}  // namespace

extern "C" {

int pfa_sparse_layer_rpb(const pfa_shape* shape, const void* Q, const void* K, const void* V, const float* bias,
                         const int32_t* I_prev, int32_t i_prev_shared, const float* A_prev,
                         int32_t K_prev, int32_t K_l, int32_t* I_out, float* A_out, float* O_out,
                         void* stream) {
    Geom g;
    int code;
    if (!geom_from_shape(shape, &g, &code)) return code;
    if (!Q || !K || !V || !I_out || !A_out || !O_out) return PFA_ERR_INVALID;
    if (K_prev < 1 || K_prev > g.N || K_l < 1 || K_l > K_prev) return PFA_ERR_INVALID;
    if (!I_prev && K_prev != g.N) return PFA_ERR_INVALID;
    if (K_prev > 1024) return PFA_ERR_UNSUPPORTED;
    if (bias && g.win == 0) return PFA_ERR_UNSUPPORTED;
    return run_sparse(g, shape->dtype, Q, K, V, bias, I_prev, i_prev_shared, A_prev, K_prev, K_l, I_out,
                      A_out, O_out, static_cast<hipStream_t>(stream));
}

int pfa_sparse_layer(const pfa_shape* shape, const void* Q, const void* K, const void* V,
                     const int32_t* I_prev, int32_t i_prev_shared, const float* A_prev,
                     int32_t K_prev, int32_t K_l, int32_t* I_out, float* A_out, float* O_out,
                     void* stream) {
    return pfa_sparse_layer_rpb(shape, Q, K, V, nullptr, I_prev, i_prev_shared, A_prev, K_prev, K_l, I_out, A_out,
                                O_out, stream);
}

int pfa_dense_layer_rpb(const pfa_shape* shape, const void* Q, const void* K, const void* V, const float* bias,
                        int32_t K1, int32_t* I_out, float* A_out, float* lse_out, float* O_out, void* stream) {
    Geom g;
    int code;
    if (!geom_from_shape(shape, &g, &code)) return code;
    if (g.win == 0) return PFA_ERR_UNSUPPORTED;
    if (!Q || !K || !V || !O_out) return PFA_ERR_INVALID;
    if (K1 < 1 || K1 > g.N) return PFA_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K1 < g.N) {
        if (!I_out || !A_out) return PFA_ERR_INVALID;
        if (lse_out) return PFA_ERR_UNSUPPORTED;
        return run_sparse(g, shape->dtype, Q, K, V, bias, nullptr, 0, nullptr, g.N, K1, I_out, A_out,
                          O_out, s);
    }
    if (g.win % 4) return PFA_ERR_UNSUPPORTED;
    if (bias && g.win % 16) return PFA_ERR_UNSUPPORTED;
    pfa::DenseArgs a;
    a.Q = Q; a.K = K; a.V = V;
    a.A_out = A_out; a.lse_out = lse_out; a.O_out = O_out;
    a.bias = bias;
    a.g = g;
    a.scale2 = (float)(1.4426950408889634 / sqrt((double)g.d));
    a.xcd_map = (n_wh(g) % 8 == 0) ? 1 : 0;
    const int64_t grid = n_wh(g) * pfa::dense_query_blocks(g.N);
    if (grid > 0x7fffffff) return PFA_ERR_UNSUPPORTED;
    hipError_t e = timed(PFA_KERNEL_DENSE, s, [&] { return pfa::launch_dense(a, shape->dtype, g.d, (int)grid, s); });
    if (e == hipSuccess && I_out)
        e = timed(PFA_KERNEL_IOTA, s, [&] { return pfa::launch_iota_rows(I_out, n_wh(g) * g.N, g.N, s); });
    return e == hipSuccess ? PFA_OK : PFA_ERR_HIP;
}

int pfa_dense_layer(const pfa_shape* shape, const void* Q, const void* K, const void* V, int32_t K1,
                    int32_t* I_out, float* A_out, float* lse_out, float* O_out, void* stream) {
    return pfa_dense_layer_rpb(shape, Q, K, V, nullptr, K1, I_out, A_out, lse_out, O_out, stream);
}

int pfa_first_two_layers(const pfa_shape* shape, int32_t shift1, int32_t shift2, const void* Q1,
                         const void* K1, const void* V1, const void* Q2, const void* K2, const void* V2,
                         int32_t K2_keep, float* lse1_out, float* O1_out, int32_t* I2_out, float* A2_out,
                         float* O2_out, void* stream) {
    Geom g;
    int code;
    if (!geom_from_shape(shape, &g, &code)) return code;
    if (shape->shift != 0) return PFA_ERR_INVALID;
    if (g.win == 0 || g.N != 1024) return PFA_ERR_UNSUPPORTED;
    if (shift1 < 0 || shift1 >= g.win || shift2 < 0 || shift2 >= g.win) return PFA_ERR_INVALID;
    if (!Q1 || !K1 || !V1 || !Q2 || !K2 || !V2 || !O1_out || !I2_out || !A2_out || !O2_out) return PFA_ERR_INVALID;
    if (K2_keep < 1 || K2_keep > g.N) return PFA_ERR_INVALID;
    if (!pfa::all_cand_dual_fits(shape->dtype, g.d)) return PFA_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const float scale2 = (float)(1.4426950408889634 / sqrt((double)g.d));
    const int xcd = (n_wh(g) % 8 == 0) ? 1 : 0;

    // layer 1: dense softmax attention, O (and optionally the log denominators) only
    pfa::DenseArgs d;
    d.Q = Q1; d.K = K1; d.V = V1;
    d.A_out = nullptr; d.lse_out = lse1_out; d.O_out = O1_out;
    d.bias = nullptr;
    d.g = g;
    d.g.shift = shift1;
    d.scale2 = scale2;
    d.xcd_map = xcd;
    const int64_t dgrid = n_wh(g) * pfa::dense_query_blocks(g.N);
    if (dgrid > 0x7fffffff) return PFA_ERR_UNSUPPORTED;
    hipError_t e = timed(PFA_KERNEL_DENSE, s, [&] { return pfa::launch_dense(d, shape->dtype, g.d, (int)dgrid, s); });
    if (e != hipSuccess) return PFA_ERR_HIP;

    // layer 2: keys from q1.k1 + q2.k2 over every slot, then the aggregation with V2
    pfa::SparseArgs a;
    a.Q = Q2; a.K = K2; a.V = V2;
    a.I_prev = nullptr; a.A_prev = nullptr;
    a.I_out = I2_out; a.A_out = A2_out; a.O_out = O2_out;
    a.g = g;
    a.g.shift = shift2;
    a.K_prev = g.N; a.K_l = K2_keep;
    a.i_shared = 0;
    a.scale2 = scale2;
    a.Q1 = Q1; a.K1 = K1; a.shift1 = shift1;
    a.bias = nullptr;
    a.xcd_map = xcd;
    a.blocks_per_wh = 2;
    a.rows_per_block = g.N / 2;
    const int64_t grid = n_wh(g) * a.blocks_per_wh;
    if (grid > 0x7fffffff) return PFA_ERR_UNSUPPORTED;
    e = timed(PFA_KERNEL_ALL_CANDIDATES, s,
              [&] { return pfa::launch_all_cand_dual(a, shape->dtype, g.d, (int)grid, s); });
    if (e == hipSuccess)
        e = timed(PFA_KERNEL_AGGREGATE, s, [&] { return pfa::launch_aggregate(a, shape->dtype, g.d, (int)grid, s); });
    return e == hipSuccess ? PFA_OK : PFA_ERR_HIP;
}

int64_t pfa_first_two_layers_backward_workspace(const pfa_shape* shape, int32_t K2_keep) {
    Geom g;
    int code;
    if (!geom_from_shape(shape, &g, &code)) return code;
    if (g.win == 0) return PFA_ERR_UNSUPPORTED;
    if (K2_keep < 1 || K2_keep > g.N) return PFA_ERR_INVALID;
    return fused_bwd_ws(g, K2_keep);
}

int pfa_first_two_layers_backward(const pfa_shape* shape, int32_t shift1, int32_t shift2, const void* Q1,
                                  const void* K1, const void* V1, const void* Q2, const void* K2, const void* V2,
                                  int32_t K2_keep, const float* lse1, const int32_t* I2, const float* A2,
                                  const float* dO1, const float* dO2, const float* dA2, float* dQ1, float* dK1,
                                  float* dV1, float* dQ2, float* dK2, float* dV2, void* workspace,
                                  int64_t workspace_bytes, void* stream) {
    Geom g;
    int code;
    if (!geom_from_shape(shape, &g, &code)) return code;
    if (shape->shift != 0) return PFA_ERR_INVALID;
    if (g.win == 0) return PFA_ERR_UNSUPPORTED;
    if (shift1 < 0 || shift1 >= g.win || shift2 < 0 || shift2 >= g.win) return PFA_ERR_INVALID;
    if (!Q1 || !K1 || !V1 || !Q2 || !K2 || !V2 || !lse1 || !I2 || !A2 || !dO1 || !dO2 || !dQ1 || !dK1 || !dV1 ||
        !dQ2 || !dK2 || !dV2 || !workspace)
        return PFA_ERR_INVALID;
    if (K2_keep < 1 || K2_keep > g.N) return PFA_ERR_INVALID;
    if (workspace_bytes < fused_bwd_ws(g, K2_keep)) return PFA_ERR_INVALID;
    if (g.win % 8 || K2_keep > 256) return PFA_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // workspace: A^1 and dA^1 at the kept slots ([wh, N, K2] each), the dense dA^1
    // ([wh, N, N]), then the two backward passes' own
    const int64_t kept_bytes = n_wh(g) * g.N * (int64_t)K2_keep * 4;
    const int64_t map_bytes = n_wh(g) * g.N * (int64_t)g.N * 4;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* A1 = reinterpret_cast<float*>(ws);
    float* dA1k = reinterpret_cast<float*>(ws + kept_bytes);
    float* dA1 = reinterpret_cast<float*>(ws + 2 * kept_bytes);
    unsigned char* ws_sparse = ws + 2 * kept_bytes + map_bytes;
    float* ws_dense = reinterpret_cast<float*>(ws_sparse + sparse_bwd_ws(g, K2_keep));

    pfa::FirstMapArgs m;
    m.Q1 = Q1; m.K1 = K1; m.I2 = I2; m.lse1 = lse1; m.A1 = A1;
    m.g = g;
    m.g.shift = shift1;
    m.K2 = K2_keep;
    m.scale2 = (float)(1.4426950408889634 / sqrt((double)g.d));
    m.blocks_per_wh = pfa::first_map_blocks(g.N);
    m.xcd_map = (n_wh(g) % 8 == 0) ? 1 : 0;
    const int64_t mgrid = n_wh(g) * m.blocks_per_wh;
    if (mgrid > 0x7fffffff) return PFA_ERR_UNSUPPORTED;
    const hipError_t e = timed(PFA_KERNEL_FIRST_MAP, s,
                               [&] { return pfa::launch_first_map(m, shape->dtype, g.d, (int)mgrid, s); });
    if (e != hipSuccess) return PFA_ERR_HIP;

    // layer 2 with its kept set as the candidate list and A^{l-1} = A^1 there: dQ2,
    // dK2, dV2 and dA^1 at the kept slots (0 at the dropped ones), spread into dense rows
    pfa_shape s2 = *shape;
    s2.shift = shift2;
    int rc = run_sparse_backward(&s2, Q2, K2, V2, nullptr, I2, A1, K2_keep, K2_keep, I2, A2, dO2, dA2, dQ2, dK2,
                                 dV2, dA1k, nullptr, ws_sparse, sparse_bwd_ws(g, K2_keep), s);
    if (rc != PFA_OK) return rc;
    pfa::SpreadArgs sp;
    sp.I = I2; sp.vals = dA1k; sp.dense = dA1;
    sp.rows = n_wh(g) * g.N;
    sp.N = g.N; sp.K = K2_keep;
    const hipError_t e2 = timed(PFA_KERNEL_FIRST_MAP, s, [&] { return pfa::launch_spread_rows(sp, s); });
    if (e2 != hipSuccess) return PFA_ERR_HIP;
    // layer 1 (dense) with that dA^1
    Geom g1 = g;
    g1.shift = shift1;
    return run_dense_backward(g1, shape->dtype, Q1, K1, V1, nullptr, lse1, dO1, dA1, dQ1, dK1, dV1, ws_dense, s);
}

int64_t pfa_sparse_layer_backward_workspace(const pfa_shape* shape, int32_t K_l) {
    Geom g;
    int code;
    if (!geom_from_shape(shape, &g, &code)) return code;
    if (K_l < 1 || K_l > g.N) return PFA_ERR_INVALID;
    return sparse_bwd_ws(g, K_l);
}

int64_t pfa_sparse_layer_backward_rpb_workspace(const pfa_shape* shape, int32_t K_l) {
    Geom g;
    int code;
    if (!geom_from_shape(shape, &g, &code)) return code;
    if (K_l < 1 || K_l > g.N) return PFA_ERR_INVALID;
    if (g.win == 0) return PFA_ERR_UNSUPPORTED;   // a bias needs window mode
    return sparse_bwd_ws(g, K_l) + dbias_part_ws(g);
}

int pfa_sparse_layer_backward(const pfa_shape* shape, const void* Q, const void* K, const void* V,
                              const int32_t* I_prev, const float* A_prev, int32_t K_prev, int32_t K_l,
                              const int32_t* I_l, const float* A_l, const float* dO, const float* dA_l,
                              float* dQ, float* dK, float* dV, float* dA_prev, void* workspace,
                              int64_t workspace_bytes, void* stream) {
    return run_sparse_backward(shape, Q, K, V, nullptr, I_prev, A_prev, K_prev, K_l, I_l, A_l, dO, dA_l, dQ, dK, dV,
                               dA_prev, nullptr, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int pfa_sparse_layer_backward_rpb(const pfa_shape* shape, const void* Q, const void* K, const void* V,
                                  const float* bias, const int32_t* I_prev, const float* A_prev, int32_t K_prev,
                                  int32_t K_l, const int32_t* I_l, const float* A_l, const float* dO,
                                  const float* dA_l, float* dQ, float* dK, float* dV, float* dA_prev, float* dbias,
                                  void* workspace, int64_t workspace_bytes, void* stream) {
    return run_sparse_backward(shape, Q, K, V, bias, I_prev, A_prev, K_prev, K_l, I_l, A_l, dO, dA_l, dQ, dK, dV,
                               dA_prev, dbias, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

int run_sparse_backward(const pfa_shape* shape, const void* Q, const void* K, const void* V, const float* bias,
                        const int32_t* I_prev, const float* A_prev, int32_t K_prev, int32_t K_l, const int32_t* I_l,
                        const float* A_l, const float* dO, const float* dA_l, float* dQ, float* dK, float* dV,
                        float* dA_prev, float* dbias, void* workspace, int64_t workspace_bytes, hipStream_t s) {
    Geom g;
    int code;
    if (!geom_from_shape(shape, &g, &code)) return code;
    if (!Q || !K || !V || !I_l || !A_l || !dO || !dQ || !dK || !dV || !workspace) return PFA_ERR_INVALID;
    if (K_prev < 1 || K_prev > g.N || K_l < 1 || K_l > K_prev) return PFA_ERR_INVALID;
    if (!I_prev && K_prev != g.N) return PFA_ERR_INVALID;
    if (dA_prev && !A_prev) return PFA_ERR_INVALID;
    if (dbias && !bias) return PFA_ERR_INVALID;
    if (workspace_bytes < sparse_bwd_ws(g, K_l) + (dbias ? dbias_part_ws(g) : 0)) return PFA_ERR_INVALID;
    if (K_l > 256) return PFA_ERR_UNSUPPORTED;
    if ((int64_t)g.N * K_l * 4 > 0x7FFFFFF0) return PFA_ERR_UNSUPPORTED;
    if (g.win == 0) {   // global mode: no bias; the dA_prev row bitmaps must fit in LDS
        if (bias || g.N > (1 << 22)) return PFA_ERR_UNSUPPORTED;
        if (dA_prev && g.N > 8192) return PFA_ERR_UNSUPPORTED;
    }
    if (!pfa::backward_dkv_sorted(shape->dtype, g.d, g.N, K_l) && !pfa::backward_dkv_mfma(g.d, g.N, K_l))
        return PFA_ERR_UNSUPPORTED;

    pfa::BackwardArgs a{};
    a.Q = Q; a.K = K; a.V = V;
    a.I_prev = I_prev; a.A_prev = A_prev;
    a.I_l = I_l; a.A_l = A_l;
    a.dO = dO; a.dA_l = dA_l;
    a.dQ = dQ; a.dK = dK; a.dV = dV; a.dA_prev = dA_prev;
    a.g_buf = static_cast<float*>(workspace);
    a.row_flags = reinterpret_cast<int32_t*>(a.g_buf + n_wh(g) * g.N * (int64_t)K_l);
    a.g = g;
    a.K_prev = K_prev; a.K_l = K_l;
    a.xcd_map = (n_wh(g) % 8 == 0) ? 1 : 0;
    a.scale = (float)(1.0 / sqrt((double)g.d));
    a.scale2 = (float)(1.4426950408889634 / sqrt((double)g.d));
    a.bias = bias;
    a.dkv_full = (int)n_wh(g);
    // rows per workgroup: a window's rows in 1 or 2 parts (K and V staged per part);
    // global mode beyond 1024 tokens stages nothing and takes 128 rows per workgroup
    a.blocks_per_wh = g.N > 1024 ? (g.N + 127) / 128 : g.N >= 512 ? 2 : 1;
    a.rows_per_block = (g.N + a.blocks_per_wh - 1) / a.blocks_per_wh;
    const int64_t rgrid = n_wh(g) * a.blocks_per_wh;
    if (rgrid > 0x7fffffff) return PFA_ERR_UNSUPPORTED;
    const int dt = shape->dtype;
    hipError_t e;
    if (pfa::backward_fused_rows(dt, g.d, g.N, K_l, dA_prev != nullptr)) {
        e = timed(PFA_KERNEL_BWD_ROWS, s, [&] { return pfa::launch_backward_rows(a, dt, g.d, true, true, (int)rgrid, s); });
    } else {
        e = timed(PFA_KERNEL_BWD_ROWS, s, [&] { return pfa::launch_backward_rows(a, dt, g.d, true, false, (int)rgrid, s); });
        if (e == hipSuccess)
            e = timed(PFA_KERNEL_BWD_ROWS, s,
                      [&] { return pfa::launch_backward_rows(a, dt, g.d, false, true, (int)rgrid, s); });
    }
    if (e == hipSuccess && dA_prev)
        e = timed(PFA_KERNEL_BWD_EXACT, s,
                  [&] { return pfa::launch_backward_exact_dap(a, dt, g.d, (int)rgrid, s); });
    if (e == hipSuccess) {
        pfa::BackwardArgs b = a;
        b.rows_per_block = g.N;
        if (pfa::backward_dkv_sorted(dt, g.d, g.N, K_l)) {
            b.blocks_per_wh = 1;
            const int64_t units = n_wh(g) * ((g.N + 1023) / 1024);   // 1024 tokens per unit
            const bool split = pfa::backward_dkv_sorted_split(dt, g.d, g.N, K_l, units, compute_units());
            // split: a dV and a dK workgroup per unit, in groups of 8 units
            const int64_t sgrid = split ? 2 * ((units + 7) / 8) * 8 : units;
            if (sgrid > 0x7fffffff) return PFA_ERR_UNSUPPORTED;
            b.dkv_units = (int)units;
            e = timed(PFA_KERNEL_BWD_SCATTER, s,
                      [&] { return pfa::launch_backward_dkv_sorted(b, dt, g.d, split, (int)sgrid, s); });
        } else {
            b.blocks_per_wh = 1;
            b.dkv_full = (int)pfa::backward_dkv_full(n_wh(g), g.N, compute_units());
            const int64_t dgrid64 = b.dkv_full + 2 * (n_wh(g) - b.dkv_full);
            if (dgrid64 > 0x7fffffff) return PFA_ERR_UNSUPPORTED;
            const int dgrid = (int)dgrid64;
            e = timed(PFA_KERNEL_BWD_SCATTER, s, [&] { return pfa::launch_backward_dkv(b, dt, g.d, dgrid, s); });
        }
    }
    if (e == hipSuccess && dbias) {
        pfa::DbiasArgs d;
        d.I_l = I_l; d.A_l = A_l; d.g_buf = a.g_buf; d.rows = nullptr;
        d.part = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + sparse_bwd_ws(g, K_l));
        d.dbias = dbias;
        d.g = g;
        d.K_l = K_l;
        e = timed(PFA_KERNEL_DBIAS, s, [&] { return pfa::launch_dbias_sparse(d, s); });
    }
    return e == hipSuccess ? PFA_OK : PFA_ERR_HIP;
}

}  // namespace

extern "C" {

int64_t pfa_dense_layer_backward_workspace(const pfa_shape* shape) {
    Geom g;
    int code;
    if (!geom_from_shape(shape, &g, &code)) return code;
    return n_wh(g) * g.N * 4;
}

int pfa_dense_layer_backward(const pfa_shape* shape, const void* Q, const void* K, const void* V, const float* bias,
                             const float* lse, const float* dO, const float* dA, float* dQ, float* dK, float* dV,
                             void* workspace, int64_t workspace_bytes, void* stream) {
    Geom g;
    int code;
    if (!geom_from_shape(shape, &g, &code)) return code;
    if (g.win == 0) return PFA_ERR_UNSUPPORTED;
    if (!Q || !K || !V || !lse || !dO || !dQ || !dK || !dV || !workspace) return PFA_ERR_INVALID;
    if (workspace_bytes < n_wh(g) * g.N * 4) return PFA_ERR_INVALID;
    if (g.win % 8) return PFA_ERR_UNSUPPORTED;
    if (bias && g.win % 16) return PFA_ERR_UNSUPPORTED;
    return run_dense_backward(g, shape->dtype, Q, K, V, bias, lse, dO, dA, dQ, dK, dV,
                              static_cast<float*>(workspace), static_cast<hipStream_t>(stream));
}

int64_t pfa_dense_layer_backward_rpb_workspace(const pfa_shape* shape) {
    Geom g;
    int code;
    if (!geom_from_shape(shape, &g, &code)) return code;
    if (g.win == 0) return PFA_ERR_UNSUPPORTED;
    return n_wh(g) * g.N * 4 + dense_dbias_rows_ws(g) + dbias_part_ws(g);
}

int pfa_dense_layer_backward_rpb(const pfa_shape* shape, const void* Q, const void* K, const void* V,
                                 const float* bias, const float* lse, const float* dO, const float* dA, float* dQ,
                                 float* dK, float* dV, float* dbias, void* workspace, int64_t workspace_bytes,
                                 void* stream) {
    Geom g;
    int code;
    if (!geom_from_shape(shape, &g, &code)) return code;
    if (g.win == 0) return PFA_ERR_UNSUPPORTED;
    if (!Q || !K || !V || !lse || !dO || !dQ || !dK || !dV || !workspace) return PFA_ERR_INVALID;
    if (dbias && !bias) return PFA_ERR_INVALID;
    const int64_t need = n_wh(g) * g.N * 4 + (dbias ? dense_dbias_rows_ws(g) + dbias_part_ws(g) : 0);
    if (workspace_bytes < need) return PFA_ERR_INVALID;
    if (g.win % 8) return PFA_ERR_UNSUPPORTED;
    if (bias && g.win % 16) return PFA_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* ws = static_cast<float*>(workspace);
    float* rows = dbias ? ws + n_wh(g) * g.N : nullptr;
    const int rc = run_dense_backward(g, shape->dtype, Q, K, V, bias, lse, dO, dA, dQ, dK, dV, ws, s, rows);
    if (rc != PFA_OK || !dbias) return rc;
    pfa::DbiasArgs d;
    d.I_l = nullptr; d.A_l = nullptr; d.g_buf = nullptr;
    d.rows = rows;
    d.part = rows + dense_dbias_rows_ws(g) / 4;
    d.dbias = dbias;
    d.g = g;
    d.K_l = 0;
    const hipError_t e = timed(PFA_KERNEL_DBIAS, s, [&] { return pfa::launch_dbias_dense(d, s); });
    return e == hipSuccess ? PFA_OK : PFA_ERR_HIP;
}

int pfa_dense_layer_backward_noalloc(const pfa_shape* shape, const void* Q, const void* K, const void* V,
                                     const float* bias, const float* lse, const float* dO, const float* dA,
                                     float* dQ, float* dK, float* dV, void* stream) {
    Geom g;
    int code;
    if (!geom_from_shape(shape, &g, &code)) return code;
    if (g.win == 0) return PFA_ERR_UNSUPPORTED;
    if (!Q || !K || !V || !lse || !dO || !dQ || !dK || !dV) return PFA_ERR_INVALID;
    if (g.win % 8) return PFA_ERR_UNSUPPORTED;
    if (bias && g.win % 16) return PFA_ERR_UNSUPPORTED;
    if (n_wh(g) * g.N * 4 > PFA_STATIC_SCRATCH_BYTES) return PFA_ERR_TOO_LARGE;
    float* Dws = nullptr;
    const int rc = static_scratch(reinterpret_cast<void**>(&Dws));
    if (rc != PFA_OK) return rc;
    return run_dense_backward(g, shape->dtype, Q, K, V, bias, lse, dO, dA, dQ, dK, dV, Dws,
                              static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

int run_dense_backward(const Geom& g, int dtype, const void* Q, const void* K, const void* V, const float* bias,
                       const float* lse, const float* dO, const float* dA, float* dQ, float* dK, float* dV,
                       float* Dws, hipStream_t s, float* dbias_rows) {
    pfa::DenseBwdArgs a;
    a.dbias_rows = dbias_rows;
    a.Q = Q; a.K = K; a.V = V;
    a.bias = bias; a.lse = lse; a.dO = dO; a.dA = dA;
    a.dQ = dQ; a.dK = dK; a.dV = dV;
    a.Dws = Dws;
    a.g = g;
    a.scale2 = (float)(1.4426950408889634 / sqrt((double)g.d));
    a.scale = (float)(1.0 / sqrt((double)g.d));
    a.xcd_map = (n_wh(g) % 8 == 0) ? 1 : 0;
    const int64_t grid = n_wh(g) * pfa::dense_bwd_blocks(g.N);
    if (grid > 0x7fffffff) return PFA_ERR_UNSUPPORTED;
    const hipError_t e = timed(PFA_KERNEL_DENSE_BWD, s,
                               [&] { return pfa::launch_dense_backward(a, dtype, g.d, (int)grid, s); });
    return e == hipSuccess ? PFA_OK : PFA_ERR_HIP;
}

}  // namespace

extern "C" {

int64_t pfa_iet_propagate_workspace(int32_t B, int32_t N, int32_t k1, int32_t k2) {
    if (B < 1 || N < 1 || k1 < 1 || k2 < 1) return PFA_ERR_INVALID;
    return (int64_t)B * N * (k1 + k2) * 4;
}

int pfa_iet_propagate(int32_t B, int32_t N, int32_t k, int32_t n_maps, const int32_t* I, const float* A,
                      int32_t k1, int32_t k2, int32_t* I_out, int32_t* count_out, void* workspace,
                      int64_t workspace_bytes, void* stream) {
    if (B < 1 || N < 1 || k < 1 || n_maps < 1) return PFA_ERR_INVALID;
    if (k2 < 1 || k1 < k2 || k1 > k) return PFA_ERR_INVALID;
    if (!I || !A || !I_out || !count_out || !workspace) return PFA_ERR_INVALID;
    if (workspace_bytes < (int64_t)B * N * (k1 + k2) * 4) return PFA_ERR_INVALID;
    if (k > 64 || N > 65536) return PFA_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    pfa::IetArgs a;
    a.I = I; a.A = A; a.I_out = I_out; a.count_out = count_out;
    a.T1 = static_cast<int32_t*>(workspace);
    a.T2 = a.T1 + (int64_t)B * N * k1;
    a.B = B; a.N = N; a.k = k; a.n_maps = n_maps; a.k1 = k1; a.k2 = k2;
    hipError_t e = timed(PFA_KERNEL_IET_RANK, s, [&] { return pfa::launch_iet_rank(a, s); });
    if (e == hipSuccess) e = timed(PFA_KERNEL_IET_UNION, s, [&] { return pfa::launch_iet_union(a, s); });
    return e == hipSuccess ? PFA_OK : PFA_ERR_HIP;
}

const char* pfa_strerror(int code) {
    switch (code) {
        case PFA_OK: return "ok";
        case PFA_ERR_INVALID: return "invalid argument";
        case PFA_ERR_UNSUPPORTED: return "unsupported configuration";
        case PFA_ERR_HIP: return "HIP runtime error";
        case PFA_ERR_TOO_LARGE: return "problem larger than the static scratch memory of a no-allocation entry point";
        default: return "unknown error code";
    }
}

int pfa_version(void) { return kVersion; }

int pfa_timing_enable(int32_t capacity) {
    if (capacity < 0 || capacity > (1 << 20)) return PFA_ERR_INVALID;
    timing_release();
    if (capacity == 0) return PFA_OK;
    g_timing.ev.assign(2 * (size_t)capacity, nullptr);
    g_timing.kind.assign(capacity, -1);
    for (hipEvent_t& e : g_timing.ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            e = nullptr;
            timing_release();
            return PFA_ERR_HIP;
        }
    }
    g_timing.on = true;
    return PFA_OK;
}

int32_t pfa_timing_count(void) { return g_timing.n; }

int pfa_timing_read(int32_t* kinds, float* ms, int32_t cap, int32_t* n_out, int32_t* dropped) {
    if (!n_out || (cap > 0 && (!kinds || !ms)) || cap < 0) return PFA_ERR_INVALID;
    Timing& t = g_timing;
    const int32_t n = t.n < cap ? t.n : cap;
    for (int32_t i = 0; i < n; ++i) {
        if (hipEventSynchronize(t.ev[2 * i + 1]) != hipSuccess) return PFA_ERR_HIP;
        if (hipEventElapsedTime(&ms[i], t.ev[2 * i], t.ev[2 * i + 1]) != hipSuccess) return PFA_ERR_HIP;
        kinds[i] = t.kind[i];
    }
    *n_out = n;
    if (dropped) *dropped = t.dropped + (t.n - n);
    t.n = 0;
    t.dropped = 0;
    return PFA_OK;
}

const char* pfa_kernel_name(int32_t kind) {
    switch (kind) {
        case PFA_KERNEL_DENSE: return "dense_layer_kernel";
        case PFA_KERNEL_ALL_CANDIDATES: return "all_cand";
        case PFA_KERNEL_SPARSE: return "sparse_layer_kernel";
        case PFA_KERNEL_SELECT: return "sparse_layer_kernel(select)";
        case PFA_KERNEL_AGGREGATE: return "aggregate";
        case PFA_KERNEL_IOTA: return "iota_rows_kernel";
        case PFA_KERNEL_BWD_ROWS: return "bwd_rows_kernel";
        case PFA_KERNEL_BWD_SCATTER: return "bwd_dkv";
        case PFA_KERNEL_IET_RANK: return "iet_rank_kernel";
        case PFA_KERNEL_IET_UNION: return "iet_union_kernel";
        case PFA_KERNEL_DENSE_BWD: return "dense_bwd";
        case PFA_KERNEL_BWD_EXACT: return "bwd_exact_dap_kernel";
        case PFA_KERNEL_DBIAS: return "dbias";
        case PFA_KERNEL_FIRST_MAP: return "first_map_kept_kernel";
        default: return "unknown";
    }
}

}  // extern "C"
