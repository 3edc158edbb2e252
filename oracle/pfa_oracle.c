/*
 * pfa_oracle.c -- plain, slow fp64 CPU reference of one progressive focused
 * attention (PFA) layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg call this code. It shares no source with the
 * HIP library and the HIP library never calls it.
 *
 * What it computes, per window-head and query slot i (sources: the Chinese paper
 * notes "Progressive Focused Transformer for Single Image Super-Resolution",
 * sections "Progressive attention across layers", "Sparse matrix multiplication"
 * and "Progressive focused resource allocation"; the index-matrix formulation of
 * "From Local Windows to Adaptive Candidates via Individualized Exploratory",
 * individualized-attention paragraph):
 *
 *   1. slot t of window (a, b) under cyclic shift s reads pixel
 *        ((a*w + t/w + s) mod H, (b*w + t%w + s) mod W);
 *      global mode: one window covering the whole map, slot = raster index;
 *   2. candidate list C_i = I^{l-1}(i) (all slots 0..N-1 when absent);
 *   3. s_ij = (q_i . k_j) / sqrt(d) for j in C_i   (the SMM: only listed pairs);
 *   4. A_cal = softmax of s over C_i;
 *   5. P = A^{l-1} (.) A_cal  (Hadamard; A^{l-1} = 1 when absent);
 *   6. P' = P / sum(P)          (Norm read as L1 row normalisation);
 *   7. keep the K_l entries with the largest P', ties to the lower index j;
 *   8. A^l = P' / sum over kept of P'   (renormalise);
 *   9. O_i = sum over kept of A^l_ij v_j, written to the pixel of slot i;
 *  10. I^l(i) lists the kept j in their C_i order, A^l aligned with it.
 * With K^l = N and no previous map this is the dense first layer.
 *
 * Everything is fp64; callers pass inputs already widened from fp32/bf16
 * (exact). No blocking, fusion or reordering beyond the steps above.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    double p;   /* P' of the candidate */
    int j;      /* candidate slot index */
    int c;      /* position in C_i */
} cand_t;

/* descending P', then ascending j */
static int cand_cmp(const void* x, const void* y) {
    const cand_t* a = (const cand_t*)x;
    const cand_t* b = (const cand_t*)y;
    if (a->p > b->p) return -1;
    if (a->p < b->p) return 1;
    return (a->j > b->j) - (a->j < b->j);
}

static int64_t pixel_of(int win, int shift, int H, int W, int wy, int wx, int t) {
    if (win == 0) return t;                     /* global mode: raster index */
    int y = (wy * win + t / win + shift) % H;
    int x = (wx * win + t % win + shift) % W;
    return (int64_t)y * W + x;
}

/* Relative position of slot j seen from slot i inside a win x win window, as
 * an index into a (2 win - 1)^2 bias table: (dy + win - 1) (2 win - 1) + (dx + win - 1)
 * with dy = i/win - j/win, dx = i%win - j%win (window-local coordinates, the same
 * under every cyclic shift). */
static int rel_index(int win, int i, int j) {
    const int dy = i / win - j / win;
    const int dx = i % win - j % win;
    return (dy + win - 1) * (2 * win - 1) + (dx + win - 1);
}

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * One PFA layer over a list of window-heads.
 *
 * Q, K, V        [B, heads, H, W, d] fp64.
 * win, shift     window side (0 = global mode, N = H*W) and cyclic shift.
 * I_prev         [B, heads or 1, nwin, N, K_prev] int32 slot indices, or NULL
 *                (then K_prev must be N and C_i = 0..N-1). i_shared = 1 means a
 *                single index matrix for all heads.
 * A_prev         [B, heads, nwin, N, K_prev] fp64 previous map, or NULL (= 1).
 * prev_compact   1: I_prev and A_prev are instead [n_wh, N, K_prev], row w of
 *                them belonging to wh_list[w] (the layout of I_out/A_out).
 * wh_list        window-head ids to compute (id = ((b*heads + h)*nwy + wy)*nwx + wx),
 *                n_wh of them; NULL means all, in order.
 * forced_keep    optional [n_wh, N, K_l]: the kept set is given instead of
 *                selected (conditional mode; steps 8-10 only use it).
 * bias           optional [heads, (2 win - 1)^2] relative position bias added
 *                to every score s_ij at index rel_index(win, i, j) (window
 *                mode only).
 * I_out, A_out   [n_wh, N, K_l] outputs (compact over wh_list).
 * key_out        optional [n_wh, N, K_prev]: ln P' per candidate in C_i order.
 * O_out          [B, heads, H, W, d]; only the pixels of listed window-heads are
 *                written.
 * Returns 0, or -1 on inconsistent sizes.
 */
int oracle_layer(int B, int heads, int H, int W, int d, int win, int shift,
                 const double* Q, const double* K, const double* V,
                 const int32_t* I_prev, int i_shared, const double* A_prev,
                 int prev_compact, int K_prev, int K_l,
                 const int64_t* wh_list, int64_t n_wh,
                 const int32_t* forced_keep, const double* bias,
                 int32_t* I_out, double* A_out, double* key_out, double* O_out) {
    const int N = win ? win * win : H * W;
    const int nwy = win ? H / win : 1, nwx = win ? W / win : 1;
    const int64_t total_wh = (int64_t)B * heads * nwy * nwx;
    if (win && (H % win || W % win)) return -1;
    if (K_l < 1 || K_l > K_prev || K_prev > N) return -1;
    if (!I_prev && K_prev != N) return -1;
    if (bias && !win) return -1;
    if (!wh_list) n_wh = total_wh;
    const double scale = 1.0 / sqrt((double)d);
    const int nrel = (2 * win - 1) * (2 * win - 1);

    int64_t w;
#pragma omp parallel for schedule(dynamic)
    for (w = 0; w < n_wh; ++w) {
        const int64_t id = wh_list ? wh_list[w] : w;
        const int wx = (int)(id % nwx);
        const int wy = (int)((id / nwx) % nwy);
        const int h = (int)((id / ((int64_t)nwx * nwy)) % heads);
        const int b = (int)(id / ((int64_t)nwx * nwy * heads));
        const int64_t plane = (int64_t)H * W * d;
        const double* Qh = Q + ((int64_t)b * heads + h) * plane;
        const double* Kh = K + ((int64_t)b * heads + h) * plane;
        const double* Vh = V + ((int64_t)b * heads + h) * plane;
        double* Oh = O_out + ((int64_t)b * heads + h) * plane;
        const int64_t win_id = (int64_t)wy * nwx + wx;
        const int64_t i_head = i_shared ? 0 : h;

        double* s = (double*)malloc(sizeof(double) * K_prev);
        double* pn = (double*)malloc(sizeof(double) * K_prev);
        char* kept = (char*)malloc(K_prev);
        cand_t* order = (cand_t*)malloc(sizeof(cand_t) * K_prev);

        for (int i = 0; i < N; ++i) {
            const double* q = Qh + pixel_of(win, shift, H, W, wy, wx, i) * d;
            const int64_t row = prev_compact ? (int64_t)w * N + i
                : (((int64_t)b * (i_shared ? 1 : heads) + i_head) * nwy * nwx + win_id) * N + i;
            const int32_t* C = I_prev ? I_prev + row * K_prev : NULL;
            const int64_t arow = prev_compact ? (int64_t)w * N + i
                : (((int64_t)b * heads + h) * nwy * nwx + win_id) * N + i;
            const double* a = A_prev ? A_prev + arow * K_prev : NULL;

            /* step 3: scaled scores over the candidate list only, plus the
             * relative position bias of (i, j) when given */
            for (int c = 0; c < K_prev; ++c) {
                const int j = C ? C[c] : c;
                const double* k = Kh + pixel_of(win, shift, H, W, wy, wx, j) * d;
                double acc = 0.0;
                for (int e = 0; e < d; ++e) acc += q[e] * k[e];
                s[c] = acc * scale;
                if (bias) s[c] += bias[(int64_t)h * nrel + rel_index(win, i, j)];
            }
            /* step 4: softmax over C_i */
            double m = s[0];
            for (int c = 1; c < K_prev; ++c) if (s[c] > m) m = s[c];
            double z = 0.0;
            for (int c = 0; c < K_prev; ++c) z += exp(s[c] - m);
            /* steps 5-6: Hadamard with the previous map, then L1 Norm */
            double sp = 0.0;
            for (int c = 0; c < K_prev; ++c) {
                const double acal = exp(s[c] - m) / z;
                pn[c] = (a ? a[c] : 1.0) * acal;
                sp += pn[c];
            }
            for (int c = 0; c < K_prev; ++c) pn[c] /= sp;
            if (key_out) {
                double* kr = key_out + ((int64_t)w * N + i) * K_prev;
                for (int c = 0; c < K_prev; ++c) kr[c] = log(pn[c]);
            }
            /* step 7: top-K_l by (descending P', ascending j) */
            memset(kept, 0, K_prev);
            if (forced_keep) {
                const int32_t* fk = forced_keep + ((int64_t)w * N + i) * K_l;
                for (int t = 0; t < K_l; ++t)
                    for (int c = 0; c < K_prev; ++c)
                        if ((C ? C[c] : c) == fk[t]) kept[c] = 1;
            } else {
                for (int c = 0; c < K_prev; ++c) {
                    order[c].p = pn[c];
                    order[c].j = C ? C[c] : c;
                    order[c].c = c;
                }
                qsort(order, K_prev, sizeof(cand_t), cand_cmp);
                for (int t = 0; t < K_l; ++t) kept[order[t].c] = 1;
            }
            /* step 8: renormalise over the kept set */
            double sk = 0.0;
            for (int c = 0; c < K_prev; ++c) if (kept[c]) sk += pn[c];
            /* steps 9-10: outputs in C_i order, O at the slot's pixel */
            double* o = Oh + pixel_of(win, shift, H, W, wy, wx, i) * d;
            for (int e = 0; e < d; ++e) o[e] = 0.0;
            int32_t* Io = I_out + ((int64_t)w * N + i) * K_l;
            double* Ao = A_out + ((int64_t)w * N + i) * K_l;
            int t = 0;
            for (int c = 0; c < K_prev; ++c) {
                if (!kept[c]) continue;
                const int j = C ? C[c] : c;
                const double aw = pn[c] / sk;
                if (t < K_l) { Io[t] = j; Ao[t] = aw; }
                ++t;
                const double* v = Vh + pixel_of(win, shift, H, W, wy, wx, j) * d;
                for (int e = 0; e < d; ++e) o[e] += aw * v[e];
            }
            for (; t < K_l; ++t) { Io[t] = -1; Ao[t] = 0.0; }
        }
        free(s); free(pn); free(kept); free(order);
    }
    return 0;
}

/*
 * Reverse-mode derivative of one PFA layer with its kept sets held fixed (the
 * selection is piecewise constant, so the kept set is a constant of the
 * backward pass). It reruns steps 1-6 and 8-10 above for each row, then walks
 * them backwards with the chain rule, one step at a time:
 *
 *   step 9  O_i = sum_kept A_c v_j      gA_c  = dA_c + dO_i . v_j,  dV_j += A_c dO_i
 *   step 8  A_c = P'_c / S (kept)       gP'_c = (gA_c - sum_kept A gA) / S, 0 if dropped
 *   step 6  P'_c = P_c / sp             gP_c  = (gP'_c - sum_c P'_c gP'_c) / sp
 *   step 5  P_c = a_c * Acal_c          gAcal_c = gP_c a_c,   dA^{l-1}_c = gP_c Acal_c
 *   step 4  Acal = softmax(s) over C_i  gs_c  = Acal_c (gAcal_c - sum_c Acal gAcal)
 *   step 3  s_c = q_i . k_j / sqrt(d)   dQ_i += gs_c k_j / sqrt(d),  dK_j += gs_c q_i / sqrt(d)
 *
 * keep      [n_wh, N, K_l] kept slot indices j of each row (the layer's I^l).
 * dO        [B, heads, H, W, d] gradient of O.
 * dA        [n_wh, N, K_l] gradient of A^l aligned with keep, or NULL (zero).
 * dQ,dK,dV  [B, heads, H, W, d]: gradients are ADDED to them (pixels of the
 *           listed window-heads only).
 * dA_prev   [n_wh, N, K_prev] gradient of A^{l-1} in C_i order (written), or
 *           NULL. Requires A_prev.
 * bias      [heads, (2 win - 1)^2] relative position bias of the forward, or NULL.
 * dbias     [heads, (2 win - 1)^2] gradient of the bias: ADDED to, or NULL.
 * Window mode or global mode with one index matrix per head; other arguments as
 * in oracle_layer. Returns 0, or -1 on inconsistent sizes or a kept slot that is
 * not a candidate.
 */
int oracle_layer_backward(int B, int heads, int H, int W, int d, int win, int shift,
                          const double* Q, const double* K, const double* V,
                          const int32_t* I_prev, const double* A_prev, int prev_compact, int K_prev, int K_l,
                          const int64_t* wh_list, int64_t n_wh, const int32_t* keep,
                          const double* dO, const double* dA, const double* bias,
                          double* dQ, double* dK, double* dV, double* dA_prev, double* dbias) {
    const int N = win ? win * win : H * W;
    const int nwy = win ? H / win : 1, nwx = win ? W / win : 1;
    const int64_t total_wh = (int64_t)B * heads * nwy * nwx;
    if (win && (H % win || W % win)) return -1;
    if (K_l < 1 || K_l > K_prev || K_prev > N) return -1;
    if (!I_prev && K_prev != N) return -1;
    if (dA_prev && !A_prev) return -1;
    if ((bias || dbias) && !win) return -1;
    if (!wh_list) n_wh = total_wh;
    const double scale = 1.0 / sqrt((double)d);
    const int nrel = (2 * win - 1) * (2 * win - 1);
    int bad = 0;

    int64_t w;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (w = 0; w < n_wh; ++w) {
        const int64_t id = wh_list ? wh_list[w] : w;
        const int wx = (int)(id % nwx);
        const int wy = (int)((id / nwx) % nwy);
        const int h = (int)((id / ((int64_t)nwx * nwy)) % heads);
        const int b = (int)(id / ((int64_t)nwx * nwy * heads));
        const int64_t plane = (int64_t)H * W * d;
        const int64_t off = ((int64_t)b * heads + h) * plane;
        const int64_t win_id = (int64_t)wy * nwx + wx;

        double* s = (double*)malloc(sizeof(double) * K_prev);
        double* acal = (double*)malloc(sizeof(double) * K_prev);
        double* pp = (double*)malloc(sizeof(double) * K_prev);     /* P' */
        double* gpp = (double*)malloc(sizeof(double) * K_prev);    /* gradient of P' */
        int* slot = (int*)malloc(sizeof(int) * K_prev);            /* position in keep, -1 dropped */
        int* pos_of = (int*)malloc(sizeof(int) * N);               /* token -> position in keep */
        for (int t = 0; t < N; ++t) pos_of[t] = -1;

        for (int i = 0; i < N; ++i) {
            const int64_t qpix = pixel_of(win, shift, H, W, wy, wx, i);
            const double* q = Q + off + qpix * d;
            const double* go = dO + off + qpix * d;
            const int64_t row = prev_compact ? (int64_t)w * N + i
                : (((int64_t)b * heads + h) * nwy * nwx + win_id) * N + i;
            const int32_t* C = I_prev ? I_prev + row * K_prev : NULL;
            const double* a = A_prev ? A_prev + row * K_prev : NULL;
            const int32_t* kp = keep + ((int64_t)w * N + i) * K_l;
            const double* dAr = dA ? dA + ((int64_t)w * N + i) * K_l : NULL;

            /* forward steps 3-6 */
            for (int c = 0; c < K_prev; ++c) {
                const int j = C ? C[c] : c;
                const double* k = K + off + pixel_of(win, shift, H, W, wy, wx, j) * d;
                double acc = 0.0;
                for (int e = 0; e < d; ++e) acc += q[e] * k[e];
                s[c] = acc * scale;
                if (bias) s[c] += bias[(int64_t)h * nrel + rel_index(win, i, j)];
            }
            double m = s[0];
            for (int c = 1; c < K_prev; ++c) if (s[c] > m) m = s[c];
            double z = 0.0;
            for (int c = 0; c < K_prev; ++c) z += exp(s[c] - m);
            double sp = 0.0;
            for (int c = 0; c < K_prev; ++c) {
                acal[c] = exp(s[c] - m) / z;
                pp[c] = (a ? a[c] : 1.0) * acal[c];
                sp += pp[c];
            }
            for (int c = 0; c < K_prev; ++c) pp[c] /= sp;
            /* step 7 replaced by the given kept set */
            int n_kept = 0;
            int ok = 1;
            for (int t = 0; t < K_l; ++t) {
                if (kp[t] < 0 || kp[t] >= N) ok = 0;
                else pos_of[kp[t]] = t;
            }
            for (int c = 0; c < K_prev; ++c) {
                const int j = C ? C[c] : c;
                slot[c] = (j >= 0 && j < N) ? pos_of[j] : -1;
                if (slot[c] >= 0) ++n_kept;
            }
            for (int t = 0; t < K_l; ++t)
                if (kp[t] >= 0 && kp[t] < N) pos_of[kp[t]] = -1;
            if (!ok || n_kept != K_l) { bad = 1; continue; }
            double S = 0.0;
            for (int c = 0; c < K_prev; ++c) if (slot[c] >= 0) S += pp[c];

            /* step 9 backwards: gA, dV; then step 8 */
            double sum_AgA = 0.0;
            for (int c = 0; c < K_prev; ++c) {
                gpp[c] = 0.0;
                if (slot[c] < 0) continue;
                const int j = C ? C[c] : c;
                const int64_t jpix = pixel_of(win, shift, H, W, wy, wx, j);
                const double* v = V + off + jpix * d;
                const double Ac = pp[c] / S;
                double gA = dAr ? dAr[slot[c]] : 0.0;
                for (int e = 0; e < d; ++e) gA += go[e] * v[e];
                double* dv = dV + off + jpix * d;
                for (int e = 0; e < d; ++e) dv[e] += Ac * go[e];
                gpp[c] = gA;           /* holds gA until the sum is known */
                sum_AgA += Ac * gA;
            }
            for (int c = 0; c < K_prev; ++c)
                if (slot[c] >= 0) gpp[c] = (gpp[c] - sum_AgA) / S;
            /* step 6 backwards */
            double sum_PgP = 0.0;
            for (int c = 0; c < K_prev; ++c) sum_PgP += pp[c] * gpp[c];
            /* steps 5 and 4 backwards: reuse gpp for gP, then s for gAcal */
            double sum_AcalgAcal = 0.0;
            for (int c = 0; c < K_prev; ++c) {
                const double gP = (gpp[c] - sum_PgP) / sp;
                if (dA_prev) dA_prev[((int64_t)w * N + i) * K_prev + c] = gP * acal[c];
                s[c] = gP * (a ? a[c] : 1.0);    /* gAcal */
                sum_AcalgAcal += acal[c] * s[c];
            }
            /* step 3 backwards (the bias gradient is summed over rows and windows
             * of each head: updates are serialised) */
            double* dq = dQ + off + qpix * d;
            for (int c = 0; c < K_prev; ++c) {
                const double gs = acal[c] * (s[c] - sum_AcalgAcal);
                const int j = C ? C[c] : c;
                if (dbias) {
#pragma omp atomic
                    dbias[(int64_t)h * nrel + rel_index(win, i, j)] += gs;
                }
                const int64_t jpix = pixel_of(win, shift, H, W, wy, wx, j);
                const double* k = K + off + jpix * d;
                double* dk = dK + off + jpix * d;
                for (int e = 0; e < d; ++e) {
                    dq[e] += gs * k[e] * scale;
                    dk[e] += gs * q[e] * scale;
                }
            }
        }
        free(s); free(acal); free(pp); free(gpp); free(slot); free(pos_of);
    }
    return bad ? -1 : 0;
}
