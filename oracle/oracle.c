/*
 * Plain CPU oracle of one MoE layer's forward pass (float64, scalar loops).
 * TEST INFRASTRUCTURE ONLY: see oracle.h for the contract and the sources.
 *
 * Deliberately simple: no blocking, no fusion, no reordering beyond what the
 * definitions state.  The only concession to run time is an OpenMP pragma on
 * independent outer loops (tokens, rows), which does not change any result:
 * every output element is computed by one thread in a fixed order.
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

int oracle_threads(void) { return omp_get_max_threads(); }

/* exact float64 value of element i of a bf16, fp32 or float64 tensor */
static double ld(int dt, const void* p, int64_t i) {
    if (dt == ORACLE_BF16) {
        uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    if (dt == ORACLE_F64) return ((const double*)p)[i];
    return (double)((const float*)p)[i];
}

double oracle_fp8_decode(uint8_t c) {
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    /* subnormal: m/8 * 2^(1-7); normal: (1 + m/8) * 2^(e-7) */
    double v = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

uint8_t oracle_fp8_encode(float x) {
    if (isnan(x)) return 0x7f;
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double a = fabs((double)x);
    if (a >= 448.0) return sign | 0x7e; /* saturate (448 is the largest finite value) */
    /* the quantum at a's binade: 2^(E-3) for a normal a in [2^E, 2^(E+1)), E >= -6; 2^-9 below */
    int E;
    frexp(a, &E); /* a = f * 2^E with f in [0.5, 1): the binade is [2^(E-1), 2^E) */
    E -= 1;
    if (E < -6) E = -6;
    double quantum = ldexp(1.0, E - 3);
    double n = nearbyint(a / quantum); /* a / quantum is exact; ties to even (default mode) */
    double v = n * quantum;             /* may step up into the next binade: still exact */
    /* encode v: find its exponent field and mantissa */
    if (v == 0.0) return sign;
    int Ev;
    frexp(v, &Ev);
    Ev -= 1;
    if (Ev < -6) return sign | (uint8_t)(v / ldexp(1.0, -9)); /* subnormal: m = v / 2^-9 */
    uint8_t m = (uint8_t)(v / ldexp(1.0, Ev - 3) - 8.0);
    return sign | (uint8_t)((Ev + 7) << 3) | m;
}

void oracle_quantize_fp8(int64_t rows, int64_t K, int dt, const void* w, uint8_t* q,
                         float* scales) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = (float)fabs(ld(dt, w, r * K + k)); /* bf16 and fp32 values are exact */
            if (a > amax) amax = a;
        }
        float scale = amax / 448.0f;
        scales[r] = scale;
        for (int64_t k = 0; k < K; ++k) {
            float v = (float)ld(dt, w, r * K + k);
            q[r * K + k] = scale == 0.0f ? 0 : oracle_fp8_encode(v / scale);
        }
    }
}

double oracle_fp4_decode(uint8_t c) {
    int sign = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    /* subnormal: m/2 * 2^(1-1); normal: (1 + m/2) * 2^(e-1) */
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -v : v;
}

uint8_t oracle_fp4_encode(float x) {
    uint8_t sign = signbit(x) ? 8 : 0;
    double a = fabs((double)x);
    if (a >= 6.0) return sign | 7; /* saturate */
    /* the quantum is 0.5 below 2, 1 in [2, 4), 2 in [4, 6] */
    double quantum = a < 2.0 ? 0.5 : a < 4.0 ? 1.0 : 2.0;
    double v = nearbyint(a / quantum) * quantum; /* ties to even multiples */
    /* codes in increasing value: 0, 0.5, 1, 1.5, 2, 3, 4, 6 */
    static const double vals[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    uint8_t code = 0;
    for (uint8_t c = 0; c < 8; ++c)
        if (vals[c] == v) code = c;
    return sign | code;
}

void oracle_quantize_mxfp4(int64_t rows, int64_t K, int dt, const void* w, uint8_t* q,
                           uint8_t* scales) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < K / 32; ++b) {
            double amax = 0.0;
            for (int64_t i = 0; i < 32; ++i) {
                double a = fabs(ld(dt, w, r * K + b * 32 + i));
                if (a > amax) amax = a;
            }
            int shared = 0;
            uint8_t sc = 127;
            if (amax > 0.0) {
                int E;
                frexp(amax, &E); /* amax = f * 2^E, f in [0.5, 1): floor(log2(amax)) = E - 1 */
                shared = E - 1 - 2;
                if (shared < -126) shared = -126;
                if (shared > 127) shared = 127;
                sc = (uint8_t)(shared + 127);
            }
            scales[r * (K / 32) + b] = sc;
            for (int64_t i = 0; i < 32; i += 2) {
                uint8_t c0 = 0, c1 = 0;
                if (amax > 0.0) {
                    c0 = oracle_fp4_encode((float)ldexp(ld(dt, w, r * K + b * 32 + i), -shared));
                    c1 = oracle_fp4_encode((float)ldexp(ld(dt, w, r * K + b * 32 + i + 1), -shared));
                }
                q[(r * K + b * 32 + i) / 2] = (uint8_t)(c0 | (c1 << 4));
            }
        }
    }
}

void oracle_dequantize_mxfp4(int64_t rows, int64_t K, const uint8_t* q, const uint8_t* scales,
                             double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = q[(r * K + k) / 2];
            uint8_t code = (k & 1) ? (byte >> 4) : (byte & 15);
            out[r * K + k] = oracle_fp4_decode(code) * ldexp(1.0, (int)scales[r * (K / 32) + k / 32] - 127);
        }
}

/* the MXFP8 rule on one block of 32 float64 values: scale code and codes */
static uint8_t mxfp8_block(const double* v, uint8_t* q) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i)
        if (fabs(v[i]) > amax) amax = fabs(v[i]);
    if (amax == 0.0) {
        for (int i = 0; i < 32; ++i) q[i] = 0;
        return 127;
    }
    int E;
    frexp(amax, &E); /* amax = f * 2^E, f in [0.5, 1): floor(log2(amax)) = E - 1 */
    int shared = E - 1 - 8;
    if (shared < -126) shared = -126;
    if (shared > 127) shared = 127;
    for (int i = 0; i < 32; ++i) q[i] = oracle_fp8_encode((float)ldexp(v[i], -shared));
    return (uint8_t)(shared + 127);
}

void oracle_quantize_mxfp8(int64_t rows, int64_t K, int dt, const void* x, uint8_t* q,
                           uint8_t* scales) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < K / 32; ++b) {
            double v[32];
            for (int i = 0; i < 32; ++i) v[i] = ld(dt, x, r * K + b * 32 + i);
            scales[r * (K / 32) + b] = mxfp8_block(v, q + r * K + b * 32);
        }
}

void oracle_dequantize_mxfp8(int64_t rows, int64_t K, const uint8_t* q, const uint8_t* scales,
                             double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * K + k] =
                oracle_fp8_decode(q[r * K + k]) * ldexp(1.0, (int)scales[r * (K / 32) + k / 32] - 127);
}

void oracle_dequantize_fp8(int64_t rows, int64_t K, const uint8_t* q, const float* scales,
                           double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * K + k] = oracle_fp8_decode(q[r * K + k]) * (double)scales[r];
}

int32_t oracle_capacity(int32_t T, int32_t k, int32_t E, double factor) {
    /* tokens per expert times the factor, counting each of the k picks */
    double c = (double)T * (double)k / (double)E * factor;
    return (int32_t)floor(c);
}

void oracle_gate(int64_t T, int64_t H, int64_t E, int dt, const void* x, const void* wg,
                 float* logits) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t e = 0; e < E; ++e) {
            double s = 0.0;
            for (int64_t h = 0; h < H; ++h) s += ld(dt, x, t * H + h) * ld(dt, wg, e * H + h);
            logits[t * E + e] = (float)s; /* one rounding to fp32 */
        }
    }
}

/* does expert a (key ka) come before expert b (key kb) in the top-k order? */
static int before(float ka, int64_t a, float kb, int64_t b) {
    if (ka > kb) return 1;
    if (ka < kb) return 0;
    return a < b; /* equal keys (+0 == -0 included): lower id first */
}

void oracle_route(int64_t T, int64_t E, int64_t k, const float* logits, const float* bias,
                  int renormalize, int bias_mode, int32_t* ids, double* w, double* margin) {
    float* key = (float*)malloc((size_t)E * sizeof(float));
    double* val = (double*)malloc((size_t)E * sizeof(double));
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t e = 0; e < E; ++e) {
            float l = logits[t * E + e];
            if (bias) l = l + bias[e]; /* a single fp32 addition */
            key[e] = l;
            taken[e] = 0;
        }
        /* selection: repeatedly take the first expert in (key desc, id asc) order */
        for (int64_t j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || before(key[e], e, key[best], best)) best = e;
            }
            taken[best] = 1;
            ids[t * k + j] = (int32_t)best;
        }
        if (margin) {
            if (k == E) {
                margin[t] = INFINITY;
            } else {
                int64_t next = -1;
                for (int64_t e = 0; e < E; ++e) {
                    if (taken[e]) continue;
                    if (next < 0 || before(key[e], e, key[next], next)) next = e;
                }
                margin[t] = (double)key[ids[t * k + k - 1]] - (double)key[next];
            }
        }
        /* the values the softmax is taken of: the keys, or with a selection-only bias the
           logits themselves */
        const int sel_only = bias && bias_mode == ORACLE_BIAS_SELECT;
        for (int64_t e = 0; e < E; ++e) val[e] = sel_only ? (double)logits[t * E + e] : (double)key[e];
        /* softmax over all experts: p_e = exp(v_e - m) / sum_e' exp(v_e' - m), m the row max */
        double m = val[0];
        for (int64_t e = 1; e < E; ++e)
            if (val[e] > m) m = val[e];
        double full = 0.0;
        for (int64_t e = 0; e < E; ++e) full += exp(val[e] - m);
        double picked = 0.0;
        for (int64_t j = 0; j < k; ++j) picked += exp(val[ids[t * k + j]] - m) / full;
        for (int64_t j = 0; j < k; ++j) {
            double p = exp(val[ids[t * k + j]] - m) / full;
            w[t * k + j] = renormalize ? p / picked : p;
        }
    }
    free(key);
    free(val);
    free(taken);
}

void oracle_load_stats(int64_t T, int64_t E, int64_t k, int32_t capacity, const int32_t* ids,
                       int32_t* raw, int64_t* ints, double* reals, float* bias_next) {
    for (int64_t e = 0; e < E; ++e) raw[e] = 0;
    for (int64_t s = 0; s < T * k; ++s)
        if (ids[s] >= 0 && ids[s] < E) raw[ids[s]]++;
    int64_t picks = 0, dropped = 0, idle = 0, hottest = 0, max_count = raw[0], min_count = raw[0];
    for (int64_t e = 0; e < E; ++e) {
        picks += raw[e];
        if (capacity >= 0 && raw[e] > capacity) dropped += raw[e] - capacity;
        if (raw[e] == 0) idle++;
        if (raw[e] > max_count) {
            max_count = raw[e];
            hottest = e;
        }
        if (raw[e] < min_count) min_count = raw[e];
    }
    double mean = (double)picks / (double)E;
    double ss = 0.0;
    for (int64_t e = 0; e < E; ++e) ss += ((double)raw[e] - mean) * ((double)raw[e] - mean);
    double stddev = sqrt(ss / (double)E);
    ints[0] = picks;
    ints[1] = dropped;
    ints[2] = max_count;
    ints[3] = hottest;
    ints[4] = min_count;
    ints[5] = idle;
    reals[0] = mean;
    reals[1] = stddev;
    reals[2] = mean > 0.0 ? stddev / mean : 0.0;
    reals[3] = mean > 0.0 ? (double)max_count / mean : 0.0;
    reals[4] = picks > 0 ? (double)dropped / (double)picks : 0.0;
    if (bias_next && capacity >= 1) {
        for (int64_t e = 0; e < E; ++e) {
            double b = ((double)capacity - (double)raw[e]) / (double)capacity;
            if (b < -1.0) b = -1.0;
            if (b > 1.0) b = 1.0;
            bias_next[e] = (float)b;
        }
    }
}

int64_t oracle_permute(int64_t T, int64_t E, int64_t k, int32_t capacity, const int32_t* ids,
                       const uint8_t* active, int32_t* raw, int32_t* counts, int32_t* offsets,
                       int32_t* row_token, int32_t* pos, uint8_t* dropped) {
    /* buckets: for each expert, its (token, slot) entries in ascending token order */
    int64_t n = T * k;
    int64_t* bucket_slot = (int64_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
    int64_t* bucket_start = (int64_t*)calloc((size_t)E + 1, sizeof(int64_t));
    int64_t* fill = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    for (int64_t e = 0; e < E; ++e) raw[e] = 0;
    for (int64_t s = 0; s < n; ++s)
        if (!active || active[s]) raw[ids[s]]++;
    for (int64_t e = 0; e < E; ++e) bucket_start[e + 1] = bucket_start[e] + raw[e];
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < k; ++j) {
            int64_t s = t * k + j;
            if (active && !active[s]) continue;
            int64_t e = ids[s];
            bucket_slot[bucket_start[e] + fill[e]++] = s;
        }
    /* capacity: keep the first `capacity` entries of each bucket */
    int64_t n_dropped = 0;
    for (int64_t s = 0; s < n; ++s) {
        pos[s] = -1;
        dropped[s] = 1;
    }
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e) {
        int64_t kept = raw[e];
        if (capacity >= 0 && kept > capacity) kept = capacity;
        counts[e] = (int32_t)kept;
        offsets[e + 1] = offsets[e] + (int32_t)kept;
        n_dropped += raw[e] - kept;
        for (int64_t r = 0; r < kept; ++r) {
            int64_t s = bucket_slot[bucket_start[e] + r];
            int32_t row = offsets[e] + (int32_t)r;
            row_token[row] = (int32_t)(s / k);
            pos[s] = row;
            dropped[s] = 0;
        }
    }
    free(bucket_slot);
    free(bucket_start);
    free(fill);
    return n_dropped;
}

static double silu(double a) { return a / (1.0 + exp(-a)); }

void oracle_expert_ffn(int64_t M, int64_t H, int64_t I, int dt_x, const void* xr, int dt_w,
                       const void* w1, const void* w3, const void* w2, double* out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        double* h = (double*)malloc((size_t)I * sizeof(double));
        for (int64_t i = 0; i < I; ++i) {
            double a = 0.0, g = 0.0;
            for (int64_t c = 0; c < H; ++c) {
                double xv = ld(dt_x, xr, m * H + c);
                a += ld(dt_w, w1, i * H + c) * xv;
                g += ld(dt_w, w3, i * H + c) * xv;
            }
            h[i] = silu(a) * g;
        }
        for (int64_t c = 0; c < H; ++c) {
            double s = 0.0;
            for (int64_t i = 0; i < I; ++i) s += ld(dt_w, w2, c * I + i) * h[i];
            out[m * H + c] = s;
        }
        free(h);
    }
}

/* quantise-dequantise n values (n % 32 == 0) through MXFP8, in place */
static void mxfp8_round_trip(double* v, int64_t n) {
    for (int64_t b = 0; b < n / 32; ++b) {
        uint8_t q[32];
        const uint8_t sc = mxfp8_block(v + b * 32, q);
        for (int i = 0; i < 32; ++i) v[b * 32 + i] = oracle_fp8_decode(q[i]) * ldexp(1.0, (int)sc - 127);
    }
}

void oracle_expert_ffn_a8(int64_t M, int64_t H, int64_t I, int dt_x, const void* xr, int dt_w,
                          const void* w1, const void* w3, const void* w2, double* out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        double* x = (double*)malloc((size_t)H * sizeof(double));
        double* h = (double*)malloc((size_t)I * sizeof(double));
        for (int64_t c = 0; c < H; ++c) x[c] = ld(dt_x, xr, m * H + c);
        mxfp8_round_trip(x, H);
        for (int64_t i = 0; i < I; ++i) {
            double a = 0.0, g = 0.0;
            for (int64_t c = 0; c < H; ++c) {
                a += ld(dt_w, w1, i * H + c) * x[c];
                g += ld(dt_w, w3, i * H + c) * x[c];
            }
            h[i] = (double)(float)(silu(a) * g);
        }
        mxfp8_round_trip(h, I);
        for (int64_t c = 0; c < H; ++c) {
            double s = 0.0;
            for (int64_t i = 0; i < I; ++i) s += ld(dt_w, w2, c * I + i) * h[i];
            out[m * H + c] = s;
        }
        free(x);
        free(h);
    }
}

void oracle_combine(int64_t T, int64_t H, int64_t k, const double* yp, const int32_t* pos,
                    const double* w, const double* ys, double* y) {
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t c = 0; c < H; ++c) {
            double s = 0.0;
            for (int64_t j = 0; j < k; ++j) {
                int32_t r = pos[t * k + j];
                if (r >= 0) s += w[t * k + j] * yp[(int64_t)r * H + c];
            }
            if (ys) s += ys[t * H + c];
            y[t * H + c] = s;
        }
    }
}

int64_t oracle_layer(int64_t T, int64_t H, int64_t E, int64_t k, int64_t I, int64_t Is,
                     int32_t capacity, int renormalize, int bias_mode, int dt, const void* x,
                     const void* wg,
                     const float* bias, const void* w1, const void* w3, const void* w2,
                     const void* ws1, const void* ws3, const void* ws2, double* y,
                     float* logits_out, int32_t* ids_out, double* w_out, int32_t* pos_out,
                     int32_t* counts_out) {
    int64_t n = T * k;
    size_t es = dt == ORACLE_BF16 ? 2 : 4;
    float* logits = (float*)malloc((size_t)(T * E > 0 ? T * E : 1) * sizeof(float));
    int32_t* ids = (int32_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(int32_t));
    double* w = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    int32_t* raw = (int32_t*)malloc((size_t)E * sizeof(int32_t));
    int32_t* counts = (int32_t*)malloc((size_t)E * sizeof(int32_t));
    int32_t* offsets = (int32_t*)malloc((size_t)(E + 1) * sizeof(int32_t));
    int32_t* row_token = (int32_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(int32_t));
    int32_t* pos = (int32_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(int32_t));
    uint8_t* dropped = (uint8_t*)malloc((size_t)(n > 0 ? n : 1));
    double* yp = (double*)malloc((size_t)(n > 0 ? n : 1) * (size_t)H * sizeof(double));
    double* ys = NULL;

    oracle_gate(T, H, E, dt, x, wg, logits);
    oracle_route(T, E, k, logits, bias, renormalize, bias_mode, ids, w, NULL);
    int64_t n_dropped =
        oracle_permute(T, E, k, capacity, ids, NULL, raw, counts, offsets, row_token, pos, dropped);

    /* each expert runs on the rows gathered for it (the packed x) */
    char* xp = (char*)malloc((size_t)(n > 0 ? n : 1) * (size_t)H * es);
    for (int64_t r = 0; r < offsets[E]; ++r)
        memcpy(xp + (size_t)r * H * es, (const char*)x + (size_t)row_token[r] * H * es, (size_t)H * es);
    for (int64_t e = 0; e < E; ++e) {
        int64_t rows = counts[e];
        if (!rows) continue;
        oracle_expert_ffn(rows, H, I, dt, xp + (size_t)offsets[e] * H * es, dt,
                          (const char*)w1 + (size_t)e * I * H * es,
                          (const char*)w3 + (size_t)e * I * H * es,
                          (const char*)w2 + (size_t)e * H * I * es, yp + (size_t)offsets[e] * H);
    }
    if (Is > 0) {
        ys = (double*)malloc((size_t)(T > 0 ? T : 1) * (size_t)H * sizeof(double));
        oracle_expert_ffn(T, H, Is, dt, x, dt, ws1, ws3, ws2, ys);
    }
    oracle_combine(T, H, k, yp, pos, w, ys, y);

    if (logits_out) memcpy(logits_out, logits, (size_t)T * E * sizeof(float));
    if (ids_out) memcpy(ids_out, ids, (size_t)n * sizeof(int32_t));
    if (w_out) memcpy(w_out, w, (size_t)n * sizeof(double));
    if (pos_out) memcpy(pos_out, pos, (size_t)n * sizeof(int32_t));
    if (counts_out) memcpy(counts_out, counts, (size_t)E * sizeof(int32_t));
    free(logits); free(ids); free(w); free(raw); free(counts); free(offsets);
    free(row_token); free(pos); free(dropped); free(yp); free(xp); free(ys);
    return n_dropped;
}
