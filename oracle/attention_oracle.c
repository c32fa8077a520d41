/*
 * CPU fp64 attention oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load or call this library.  It shares no code with the GPU path.
 *
 * What it computes is the plain definition the ring method must reproduce:
 * "Ring Attention" (Ultralytics glossary), section "How ring attention works":
 * the ring's result equals full softmax attention softmax(q k^T / sqrt(d)) v,
 * exactly up to rounding; the same passage says production kernels subtract a
 * running maximum before exponentiating, which is what the max M below is.
 * The causal rule is the `is_causal=True` mask of "Context Parallelism"
 * (Ultralytics glossary), section "Practical use and trade-offs": a key is
 * allowed iff its global position is <= the query's global position.
 *
 * For one query row q with global position tq, keys/values (k_c, v_c) with
 * global positions pc, scale sigma (1/sqrt(d) unless given):
 *     C     = { c : !causal or pc <= tq }          (allowed keys)
 *     s_c   = sigma * sum_k q[k] * k_c[k]           (c in C)
 *     M     = max_{c in C} s_c                      (-inf if C is empty)
 *     Z     = sum_{c in C} exp(s_c - M)             (0 if C is empty)
 *     N     = sum_{c in C} exp(s_c - M) * v_c       (numerator, 0 if C empty)
 *     O     = N / Z                                 (0 if C is empty)
 *     lse   = M + ln Z                              (-inf if C is empty)
 * (M, Z, N) is the "partial" of this key set: the same triple a blockwise
 * kernel returns for one key block.  Everything is fp64; inputs are read as
 * binary32 or bfloat16 bit patterns and widened exactly.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC attention_oracle.c -o libra_oracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

static double load_elem(const void* base, int dtype, int64_t i) {
    if (dtype == ORACLE_F32) return (double)((const float*)base)[i];
    uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/*
 * Rows r in [0, n_rows): query vector q[r*d .. r*d+d), position q_pos[r].
 * Keys c in [0, n_keys): k[c*d ..], v[c*d ..], position k_pos[c] (k_pos may be
 * NULL, meaning position c).  Any output pointer may be NULL.
 * o_num, o: [n_rows, d]; m, l, lse: [n_rows].  Returns 0, -1 on bad arguments,
 * -2 if scratch memory could not be allocated.
 */
int ra_oracle_rows(int64_t d, double scale, int causal, int dtype, int64_t n_rows,
                   const void* q, const int64_t* q_pos, int64_t n_keys, const void* k,
                   const void* v, const int64_t* k_pos, double* o_num, double* m, double* l,
                   double* o, double* lse) {
    if (d <= 0 || n_rows < 0 || n_keys < 0 || !q || (n_keys > 0 && (!k || !v))) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    if (causal && !q_pos) return -1;
    if (!(scale > 0.0)) scale = 1.0 / sqrt((double)d);
    int failed = 0;

#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1));
        double* qr = (double*)malloc(sizeof(double) * (size_t)d);
        double* num = (double*)malloc(sizeof(double) * (size_t)d);
        unsigned char* allowed = (unsigned char*)malloc((size_t)(n_keys > 0 ? n_keys : 1));
        if (!s || !qr || !num || !allowed) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!s || !qr || !num || !allowed) continue;
            for (int64_t j = 0; j < d; ++j) qr[j] = load_elem(q, dtype, r * d + j);
            /* scores over the allowed keys, and their maximum */
            double M = -INFINITY;
            int64_t n_allowed = 0;
            for (int64_t c = 0; c < n_keys; ++c) {
                const int64_t pc = k_pos ? k_pos[c] : c;
                allowed[c] = (unsigned char)(!causal || pc <= q_pos[r]);
                if (!allowed[c]) continue;
                double dot = 0.0;
                for (int64_t j = 0; j < d; ++j) dot += qr[j] * load_elem(k, dtype, c * d + j);
                s[c] = scale * dot;
                if (s[c] > M) M = s[c];
                ++n_allowed;
            }
            /* Z = sum exp(s - M);  N = sum exp(s - M) v */
            double Z = 0.0;
            for (int64_t j = 0; j < d; ++j) num[j] = 0.0;
            if (n_allowed > 0) {
                for (int64_t c = 0; c < n_keys; ++c) {
                    if (!allowed[c]) continue;
                    const double w = exp(s[c] - M);
                    Z += w;
                    for (int64_t j = 0; j < d; ++j) num[j] += w * load_elem(v, dtype, c * d + j);
                }
            }
            if (o_num)
                for (int64_t j = 0; j < d; ++j) o_num[r * d + j] = num[j];
            if (m) m[r] = M;
            if (l) l[r] = Z;
            if (o)
                for (int64_t j = 0; j < d; ++j) o[r * d + j] = n_allowed ? num[j] / Z : 0.0;
            if (lse) lse[r] = n_allowed ? M + log(Z) : -INFINITY;
        }
        free(s);
        free(qr);
        free(num);
        free(allowed);
    }
    return failed ? -2 : 0;
}

/*
 * Gradients of the same attention -- TEST INFRASTRUCTURE ONLY.
 *
 * The pages run the backward pass: "Context Parallelism" (Ultralytics
 * glossary), section "Practical use and trade-offs", marks q, k, v as
 * requiring gradients and back-propagates a loss through the causal attention
 * output.  For O = softmax(S) V with S = sigma Q K^T (masked entries excluded)
 * and an upstream gradient dO = dL/dO, the chain rule gives, per query row t
 * and allowed key c:
 *     p_tc   = exp(s_tc - lse_t)                     (the softmax weights)
 *     dp_tc  = dO_t . v_c                            (dL/dp_tc)
 *     D_t    = sum_{c in C_t} p_tc dp_tc             (= dO_t . O_t)
 *     ds_tc  = p_tc (dp_tc - D_t)                    (dL/ds_tc, softmax Jacobian)
 *     dQ_t   = sigma sum_{c in C_t} ds_tc k_c
 *     dK_c   = sigma sum_{t : c in C_t} ds_tc q_t
 *     dV_c   = sum_{t : c in C_t} p_tc dO_t
 * Pass 1 runs over query rows (lse_t, D_t, dQ_t), pass 2 over keys (dK_c,
 * dV_c) with the lse_t and D_t of pass 1; both evaluate the definitions above
 * directly in fp64.
 *
 * lse_in / delta_in (fp64 [n_rows], may be NULL): use these lse_t and D_t
 * instead of computing them over the given keys -- this gives one key block's
 * share of the gradients when lse and D belong to the row's full key set.
 * dout has the dtype of q, k, v.  dq [n_rows, d], dk, dv [n_keys, d],
 * lse_out, delta_out [n_rows]: any may be NULL.  Returns 0, -1 on bad
 * arguments, -2 if scratch memory could not be allocated.
 */
int ra_oracle_grads(int64_t d, double scale, int causal, int dtype, int64_t n_rows,
                    const void* q, const int64_t* q_pos, const void* dout, int64_t n_keys,
                    const void* k, const void* v, const int64_t* k_pos, const double* lse_in,
                    const double* delta_in, double* dq, double* dk, double* dv, double* lse_out,
                    double* delta_out) {
    if (d <= 0 || n_rows < 0 || n_keys < 0 || (n_rows > 0 && (!q || !dout)) ||
        (n_keys > 0 && (!k || !v)))
        return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    if (causal && !q_pos) return -1;
    if (!(scale > 0.0)) scale = 1.0 / sqrt((double)d);
    double* lse = (double*)malloc(sizeof(double) * (size_t)(n_rows > 0 ? n_rows : 1));
    double* delta = (double*)malloc(sizeof(double) * (size_t)(n_rows > 0 ? n_rows : 1));
    if (!lse || !delta) {
        free(lse);
        free(delta);
        return -2;
    }
    int failed = 0;

    /* pass 1: per query row */
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1));
        double* qr = (double*)malloc(sizeof(double) * (size_t)d);
        double* gr = (double*)malloc(sizeof(double) * (size_t)d);
        double* acc = (double*)malloc(sizeof(double) * (size_t)d);
        if (!s || !qr || !gr || !acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!s || !qr || !gr || !acc) continue;
            for (int64_t j = 0; j < d; ++j) {
                qr[j] = load_elem(q, dtype, r * d + j);
                gr[j] = load_elem(dout, dtype, r * d + j);
            }
            double M = -INFINITY;
            for (int64_t c = 0; c < n_keys; ++c) {
                const int64_t pc = k_pos ? k_pos[c] : c;
                if (causal && pc > q_pos[r]) continue;
                double dot = 0.0;
                for (int64_t j = 0; j < d; ++j) dot += qr[j] * load_elem(k, dtype, c * d + j);
                s[c] = scale * dot;
                if (s[c] > M) M = s[c];
            }
            double L;
            if (lse_in) {
                L = lse_in[r];
            } else if (M == -INFINITY) {
                L = -INFINITY;
            } else {
                double Z = 0.0;
                for (int64_t c = 0; c < n_keys; ++c) {
                    const int64_t pc = k_pos ? k_pos[c] : c;
                    if (causal && pc > q_pos[r]) continue;
                    Z += exp(s[c] - M);
                }
                L = M + log(Z);
            }
            /* D_t = sum p dp (or given) */
            double D = 0.0;
            if (delta_in) {
                D = delta_in[r];
            } else if (L != -INFINITY) {
                for (int64_t c = 0; c < n_keys; ++c) {
                    const int64_t pc = k_pos ? k_pos[c] : c;
                    if (causal && pc > q_pos[r]) continue;
                    double dp = 0.0;
                    for (int64_t j = 0; j < d; ++j) dp += gr[j] * load_elem(v, dtype, c * d + j);
                    D += exp(s[c] - L) * dp;
                }
            }
            /* dQ_t = sigma sum ds k */
            for (int64_t j = 0; j < d; ++j) acc[j] = 0.0;
            if (L != -INFINITY) {
                for (int64_t c = 0; c < n_keys; ++c) {
                    const int64_t pc = k_pos ? k_pos[c] : c;
                    if (causal && pc > q_pos[r]) continue;
                    double dp = 0.0;
                    for (int64_t j = 0; j < d; ++j) dp += gr[j] * load_elem(v, dtype, c * d + j);
                    const double p = exp(s[c] - L);
                    const double ds = p * (dp - D);
                    for (int64_t j = 0; j < d; ++j) acc[j] += ds * load_elem(k, dtype, c * d + j);
                }
            }
            if (dq)
                for (int64_t j = 0; j < d; ++j) dq[r * d + j] = scale * acc[j];
            lse[r] = L;
            delta[r] = D;
        }
        free(s);
        free(qr);
        free(gr);
        free(acc);
    }

    /* pass 2: per key */
    if (!failed && (dk || dv)) {
#pragma omp parallel
        {
            double* kr = (double*)malloc(sizeof(double) * (size_t)d);
            double* vr = (double*)malloc(sizeof(double) * (size_t)d);
            double* ak = (double*)malloc(sizeof(double) * (size_t)d);
            double* av = (double*)malloc(sizeof(double) * (size_t)d);
            if (!kr || !vr || !ak || !av) {
#pragma omp atomic write
                failed = 1;
            }
#pragma omp for schedule(dynamic, 1)
            for (int64_t c = 0; c < n_keys; ++c) {
                if (!kr || !vr || !ak || !av) continue;
                const int64_t pc = k_pos ? k_pos[c] : c;
                for (int64_t j = 0; j < d; ++j) {
                    kr[j] = load_elem(k, dtype, c * d + j);
                    vr[j] = load_elem(v, dtype, c * d + j);
                    ak[j] = 0.0;
                    av[j] = 0.0;
                }
                for (int64_t r = 0; r < n_rows; ++r) {
                    if (causal && pc > q_pos[r]) continue;
                    if (lse[r] == -INFINITY) continue;
                    double dot = 0.0, dp = 0.0;
                    for (int64_t j = 0; j < d; ++j) {
                        dot += load_elem(q, dtype, r * d + j) * kr[j];
                        dp += load_elem(dout, dtype, r * d + j) * vr[j];
                    }
                    const double p = exp(scale * dot - lse[r]);
                    const double ds = p * (dp - delta[r]);
                    for (int64_t j = 0; j < d; ++j) {
                        av[j] += p * load_elem(dout, dtype, r * d + j);
                        ak[j] += ds * load_elem(q, dtype, r * d + j);
                    }
                }
                for (int64_t j = 0; j < d; ++j) {
                    if (dk) dk[c * d + j] = scale * ak[j];
                    if (dv) dv[c * d + j] = av[j];
                }
            }
            free(kr);
            free(vr);
            free(ak);
            free(av);
        }
    }
    if (lse_out)
        for (int64_t r = 0; r < n_rows; ++r) lse_out[r] = lse[r];
    if (delta_out)
        for (int64_t r = 0; r < n_rows; ++r) delta_out[r] = delta[r];
    free(lse);
    free(delta);
    return failed ? -2 : 0;
}
