/*
 * Float64 C twin of the WKV oracle (oracle/wkv_ref.py), for workloads too
 * large for the numpy loops: the decode-state seeding of 32 x 256 x 4096
 * lanes, the 1000 decode steps of every one of those lanes, and the CPU
 * baseline timing.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py load this library; the HIP product path never
 * links or calls it, and it shares no code with it.
 *
 * It computes the same plain (unscaled) float64 recurrences as the numpy
 * oracle, one lane (b, c) at a time, lanes spread over OpenMP threads:
 *
 *   "RWKV - 把 RNN 重新带回 Transformer 时代的线性大模型", sections
 *   "一句话总结" and "关键设计 2：WKV 算子":
 *       y_t = (A_{t-1} + e^{u+k_t} v_t) / (B_{t-1} + e^{u+k_t})
 *       A_t = e^{-w} A_{t-1} + e^{k_t} v_t,  B_t = e^{-w} B_{t-1} + e^{k_t}
 *   with A_0 = B_0 = 0.  The backward is the derivative of the weighted sum
 *   of "RWKV（Receptance Weighted Key Value）概念", section 3.2, written as
 *   the reverse recurrences documented in wkv_ref.py (wkv_backward_ref).
 *
 * Inputs are float32 arrays (exact copies of the fp32 or bf16-rounded values
 * the GPU consumes) and are promoted to double; every sum is double.
 * Layout: k, v, gy, y, dk, dv are [B, T, C] with C fastest; w, u are [C].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int wkv_ref_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Forward.  y (nullable) receives [B,T,C] doubles; A_out, B_out (nullable)
 * receive the final plain sums [B,C].  Returns the number of threads used. */
int wkv_ref_forward(int64_t B, int64_t T, int64_t C, const float* w,
                    const float* u, const float* k, const float* v, double* y,
                    double* A_out, double* B_out, int nthreads) {
    int used = 1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
    {
#pragma omp single
        used = omp_get_num_threads();
#pragma omp for collapse(2) schedule(static)
#endif
        for (int64_t b = 0; b < B; ++b) {
            for (int64_t c = 0; c < C; ++c) {
                const double d = exp(-(double)w[c]);
                const double eu = exp((double)u[c]);
                double A = 0.0, Bs = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    const int64_t i = (b * T + t) * C + c;
                    const double ek = exp((double)k[i]);
                    const double cur = eu * ek;
                    const double vt = (double)v[i];
                    if (y) y[i] = (A + cur * vt) / (Bs + cur);
                    A = d * A + ek * vt;
                    Bs = d * Bs + ek;
                }
                if (A_out) A_out[b * C + c] = A;
                if (B_out) B_out[b * C + c] = Bs;
            }
        }
#ifdef _OPENMP
    }
#endif
    return used;
}

/* Backward of L = sum(gy * y).  dk, dv: [B,T,C] doubles; dw, du: [C] doubles
 * (summed over b and t).  Returns the number of threads used, or -1 when a
 * scratch allocation fails. */
int wkv_ref_backward(int64_t B, int64_t T, int64_t C, const float* w,
                     const float* u, const float* k, const float* v,
                     const float* gy, double* dk, double* dv, double* dw,
                     double* du, int nthreads) {
    int used = 1, failed = 0;
    double* dw_lane = (double*)calloc((size_t)(B * C), sizeof(double));
    double* du_lane = (double*)calloc((size_t)(B * C), sizeof(double));
    if (!dw_lane || !du_lane) {
        free(dw_lane);
        free(du_lane);
        return -1;
    }
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
    {
#pragma omp single
        used = omp_get_num_threads();
#endif
        double* ys = (double*)malloc((size_t)T * sizeof(double));
        double* Ds = (double*)malloc((size_t)T * sizeof(double));
        if (!ys || !Ds) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for collapse(2) schedule(static)
#endif
        for (int64_t b = 0; b < B; ++b) {
            for (int64_t c = 0; c < C; ++c) {
                if (!ys || !Ds) continue;
                const double d = exp(-(double)w[c]);
                const double eu = exp((double)u[c]);
                double A = 0.0, Bs = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    const int64_t i = (b * T + t) * C + c;
                    const double ek = exp((double)k[i]);
                    const double cur = eu * ek;
                    const double vt = (double)v[i];
                    Ds[t] = Bs + cur;
                    ys[t] = (A + cur * vt) / Ds[t];
                    A = d * A + ek * vt;
                    Bs = d * Bs + ek;
                }
                double G = 0.0, H = 0.0, Gp = 0.0, Hp = 0.0;
                double dwl = 0.0, dul = 0.0;
                for (int64_t t = T - 1; t >= 0; --t) {
                    const int64_t i = (b * T + t) * C + c;
                    const double ek = exp((double)k[i]);
                    const double pi = eu * ek / Ds[t];
                    const double gt = (double)gy[i], vt = (double)v[i];
                    const double yt = ys[t];
                    const double cur_k = gt * pi * (vt - yt);
                    dv[i] = gt * pi + ek * G;
                    dk[i] = cur_k + ek * (vt * G - H);
                    dul += cur_k;
                    dwl -= ek * (vt * Gp - Hp);
                    Gp = d * (Gp + G);
                    Hp = d * (Hp + H);
                    G = d * G + gt / Ds[t];
                    H = d * H + gt * yt / Ds[t];
                }
                dw_lane[b * C + c] = dwl;
                du_lane[b * C + c] = dul;
            }
        }
        free(ys);
        free(Ds);
#ifdef _OPENMP
    }
#endif
    for (int64_t c = 0; c < C; ++c) {
        double sw = 0.0, su = 0.0;
        for (int64_t b = 0; b < B; ++b) {
            sw += dw_lane[b * C + c];
            su += du_lane[b * C + c];
        }
        dw[c] = sw;
        du[c] = su;
    }
    free(dw_lane);
    free(du_lane);
    return failed ? -1 : used;
}

/* bf16 bits -> float32 value (exact: bf16 is the top half of a float32). */
static inline float bf16_value(uint16_t x) {
    union {
        uint32_t u;
        float f;
    } c;
    c.u = (uint32_t)x << 16;
    return c.f;
}

/* One recurrent-mode (decode) token for L x B x C lanes, on the plain float64
 * sums of the state, A (numerator) and B (denominator):
 *
 *   "RWKV - 把 RNN 重新带回 Transformer 时代的线性大模型", section
 *   "关键设计 4" (recurrent mode: the output reads the state before the
 *   token, the token then enters with its own weight) and "关键设计 2":
 *       y  = (A + e^{u+k} v) / (B + e^{u+k})
 *       A' = e^{-w} A + e^{k} v,      B' = e^{-w} B + e^{k}
 *
 * The same plain recurrence as wkv_ref_forward (so T steps from A = B = 0
 * are that forward), without the running-max rescale of the numpy step
 * oracle: these sums stay far inside float64's range for the decode
 * workloads (|k| of a few units).
 *
 * w, u: [L, C] float32.  k, v: [L, B, C] as float32 values (bf16 == 0) or as
 * bf16 bits (bf16 != 0).  A, Bs: [L, B, C] doubles, read and updated in
 * place.  y (nullable): [L, B, C] doubles.  Returns the number of threads
 * used, or -1 when a scratch allocation fails. */
int wkv_ref_step(int64_t L, int64_t B, int64_t C, const float* w, const float* u, const void* k, const void* v,
                 int bf16, double* A, double* Bs, double* y, int nthreads) {
    int used = 1;
    double* dtab = (double*)malloc((size_t)(L * C) * sizeof(double));
    double* eutab = (double*)malloc((size_t)(L * C) * sizeof(double));
    if (!dtab || !eutab) {
        free(dtab);
        free(eutab);
        return -1;
    }
    for (int64_t i = 0; i < L * C; ++i) {  /* per (layer, channel): e^{-w}, e^{u} */
        dtab[i] = exp(-(double)w[i]);
        eutab[i] = exp((double)u[i]);
    }
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
    {
#pragma omp single
        used = omp_get_num_threads();
#pragma omp for collapse(2) schedule(static)
#endif
        for (int64_t l = 0; l < L; ++l) {
            for (int64_t b = 0; b < B; ++b) {
                for (int64_t c = 0; c < C; ++c) {
                    const int64_t i = (l * B + b) * C + c;
                    const double d = dtab[l * C + c];
                    const double eu = eutab[l * C + c];
                    const double kt = bf16 ? (double)bf16_value(((const uint16_t*)k)[i]) : (double)((const float*)k)[i];
                    const double vt = bf16 ? (double)bf16_value(((const uint16_t*)v)[i]) : (double)((const float*)v)[i];
                    const double ek = exp(kt);
                    const double cur = eu * ek;
                    if (y) y[i] = (A[i] + cur * vt) / (Bs[i] + cur);
                    A[i] = d * A[i] + ek * vt;
                    Bs[i] = d * Bs[i] + ek;
                }
            }
        }
#ifdef _OPENMP
    }
#endif
    free(dtab);
    free(eutab);
    return used;
}
