/*
 * sage_oracle.c -- plain, slow CPU oracle for the quantized attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load
 * this file or the library built from it; only the tests, the package's smoke
 * check and the benchmark's CPU-baseline leg do.  It shares no code, header,
 * table or constant generator with the HIP kernels.
 *
 * Sources (three web pages on SageAttention; cited by title and section):
 *   [guide]  "SageAttention deployment guide: from environment to multi-GPU
 *            tuning, 2-5x faster attention" (pwwt.cn/news/4103508)
 *   [amd-wsl] "Using SageAttention on AMD cards without installing the HIP SDK"
 *            (trdm.cn/news/481702)
 *   [amd-9070] "SageAttention 2.2.0 on the RX 9070 XT" (pnsm.cn/news/1834815)
 *
 * What the pages fix: Q and K are quantized to INT8 with per-block / per-warp /
 * per-thread scale factors and QK^T is an 8-bit integer product ([guide] sec. 1,
 * first bullet; sec. 4.2 table, qk_quant_gran); V is lowered to FP8 and P.V is
 * accumulated in FP16/FP32 ([guide] sec. 1, second bullet; sec. 4 dispatch
 * table); the output stays FP16/BF16 ([guide] sec. 1, third bullet); the
 * softmax is computed block by block as in FlashAttention, each block getting
 * its own value range before it is compressed ([amd-9070] sec. 2).  Where the
 * pages are silent (formulae, rounding, group shapes, P precision) this file
 * follows the readings listed in the repository's design notes; each function
 * says which.
 *
 * Precision: every value that is rounded to a code (INT8 codes of Q and K, FP8
 * codes of V and P) is formed in fp32, with one rounding per arithmetic step
 * as written, so that codes are defined to the bit and can be compared; every
 * accumulation that decides no code (means, P.V, row sums) is carried in fp64.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Round-to-nearest-even into a binary floating-point format with `mbits`
 * stored mantissa bits and minimum normal exponent `emin`.  Values must
 * already lie within the format's finite range.  For |x| in [2^e, 2^(e+1))
 * with e >= emin the spacing of representable values is 2^(e - mbits); below
 * 2^emin (subnormals) it is 2^(emin - mbits).  Dividing by a power of two is
 * exact, and nearbyint() rounds half to even under the default rounding mode,
 * which makes the result's last mantissa bit even on ties.                   */
static double fmt_rne(double x, int mbits, int emin) {
    if (x == 0.0) return x;
    double ax = fabs(x);
    int e2;
    frexp(ax, &e2);               /* ax = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;               /* ax in [2^e, 2^(e+1)) */
    if (e < emin) e = emin;
    double quantum = ldexp(1.0, e - mbits);
    double r = nearbyint(ax / quantum) * quantum;
    return x < 0 ? -r : r;
}

/* OCP E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, largest
 * finite value 448, no infinities ([guide] sec. 1 names FP8 for V; the FN
 * variant is the one whose largest value is 448).                            */
#define E4M3_MAX 448.0
static double e4m3_value(double x) {               /* x already in [-448, 448] */
    return fmt_rne(x, 3, -6);
}

/* Code byte of an E4M3FN value v that is exactly representable.  The sign bit
 * is the sign bit of the input, as for any IEEE-style conversion: negative
 * values that round to zero, and -0.0 itself, encode as 0x80.                */
static uint8_t e4m3_code_of(double x_before_rounding, double v) {
    uint8_t sign = signbit(x_before_rounding) ? 0x80 : 0x00;
    double av = fabs(v);
    if (av == 0.0) return sign;
    int e2;
    frexp(av, &e2);
    int e = e2 - 1;
    if (e < -6) {                                  /* subnormal: m * 2^-9 */
        int m = (int)(av / ldexp(1.0, -9));
        return (uint8_t)(sign | m);
    }
    int m = (int)(av / ldexp(1.0, e - 3)) - 8;     /* 0..7 */
    return (uint8_t)(sign | ((e + 7) << 3) | m);
}

/* exported codec helpers (pinned by the tests against a library cast) */
uint8_t oracle_e4m3_encode(float x) {
    double c = x;
    if (c > E4M3_MAX) c = E4M3_MAX;
    if (c < -E4M3_MAX) c = -E4M3_MAX;
    return e4m3_code_of(c, e4m3_value(c));
}

float oracle_e4m3_decode(uint8_t code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(8.0 + m, e - 10);
    return (float)(s ? -v : v);
}

/* fp32 -> fp16 / bf16 value (round to nearest even).  fp16: 10 mantissa bits,
 * emin -14; bf16: 7 mantissa bits, emin -126.                                 */
float oracle_round_half(float x, int is_bf16) {
    return is_bf16 ? (float)fmt_rne(x, 7, -126) : (float)fmt_rne(x, 10, -14);
}

/* array forms of the codec helpers */
void oracle_e4m3_encode_array(const float* x, int64_t n, uint8_t* codes) {
    for (int64_t i = 0; i < n; ++i) codes[i] = oracle_e4m3_encode(x[i]);
}

void oracle_round_half_array(const float* x, int64_t n, int is_bf16, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_half(x[i], is_bf16);
}

/* ------------------------------------------------------------------------ */
/* Symmetric INT8 group quantizer ([guide] sec. 1, first bullet: INT8 with
 * per-block/per-thread scales; [amd-9070] sec. 2: each block gets its own
 * value range).  Reading: range +-127, scale = amax/127 stored in fp32,
 * code = rint(x * fl32(127/amax)) with ties to even; an all-zero group has
 * scale 0 and codes 0.
 *
 * x:     rows x dp fp32 matrix (row-major); rows beyond `n_valid` are ignored
 *        and their codes set to 0.
 * group: number of consecutive rows sharing one scale; groups start at row 0.
 * codes: rows x dp int8; scales: ceil(rows/group) floats.                    */
void oracle_quant_int8_rows(const float* x, int rows, int n_valid, int dp, int group,
                            int8_t* codes, float* scales) {
    int ngroups = (rows + group - 1) / group;
    memset(codes, 0, (size_t)rows * dp);
    for (int g = 0; g < ngroups; ++g) {
        int r0 = g * group, r1 = r0 + group;
        if (r1 > n_valid) r1 = n_valid;
        float amax = 0.0f;
        for (int r = r0; r < r1; ++r)
            for (int c = 0; c < dp; ++c) {
                float a = fabsf(x[(size_t)r * dp + c]);
                if (a > amax) amax = a;
            }
        if (amax == 0.0f || r1 <= r0) { scales[g] = 0.0f; continue; }
        volatile float scale = amax / 127.0f;   /* fp32 division */
        volatile float inv = 127.0f / amax;
        scales[g] = scale;
        for (int r = r0; r < r1; ++r)
            for (int c = 0; c < dp; ++c) {
                volatile float t = x[(size_t)r * dp + c] * inv;   /* fp32 product */
                float q = nearbyintf(t);
                if (q > 127.0f) q = 127.0f;
                if (q < -127.0f) q = -127.0f;
                codes[(size_t)r * dp + c] = (int8_t)q;
            }
    }
}

/* ------------------------------------------------------------------------ */
/* FP8 quantization of V, one scale per channel over the valid rows
 * ([guide] sec. 1, second bullet: V lowered to FP8).  Reading: per-channel
 * scale amax_c/448 (the channel scale then factors out of the sum over keys),
 * code = E4M3FN_rne(clamp(fl32(v * fl32(448/amax_c)), +-448)); an all-zero
 * channel has scale 0 and codes 0.
 * v: n x dp fp32 (already smoothed if smooth_v); codes: n x dp; scales: dp.  */
void oracle_quant_v_fp8(const float* v, int n, int dp, uint8_t* codes, float* scales) {
    for (int c = 0; c < dp; ++c) {
        float amax = 0.0f;
        for (int r = 0; r < n; ++r) {
            float a = fabsf(v[(size_t)r * dp + c]);
            if (a > amax) amax = a;
        }
        if (amax == 0.0f) {
            scales[c] = 0.0f;
            for (int r = 0; r < n; ++r) codes[(size_t)r * dp + c] = 0;
            continue;
        }
        volatile float scale = amax / 448.0f;
        volatile float inv = 448.0f / amax;
        scales[c] = scale;
        for (int r = 0; r < n; ++r) {
            volatile float t = v[(size_t)r * dp + c] * inv;
            double tc = t;
            if (tc > E4M3_MAX) tc = E4M3_MAX;
            if (tc < -E4M3_MAX) tc = -E4M3_MAX;
            codes[(size_t)r * dp + c] = e4m3_code_of(tc, e4m3_value(tc));
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Quantized attention for selected query rows of one (sequence, head) pair,
 * following the method's steps in order:
 *   scores  S_ij = sum_c q8_ic k8_jc in exact integer arithmetic
 *           ([guide] sec. 1: QK^T by 8-bit integer multiplication);
 *   dequant c_i = fl32(fl32(qscale_i * sm_scale) * log2(e)) and
 *           s_ij = fl32(fl32(S_ij * kscale_j) * c_i), the score in log2 units;
 *   online softmax over key tiles of `bk` keys in ascending order, as in
 *           FlashAttention ([amd-9070] sec. 2: the softmax is computed block
 *           by block, each block with its own value range):
 *             m' = max(m, largest visible s_ij of the tile),
 *             the running sums are rescaled by alpha = 2^(m - m') when the
 *             maximum moves (the first tile starts from zero sums),
 *             x_ij = fl32(s_ij - m'),  p_ij = fl32(2^x_ij) <= 1;
 *   P       the P.V operand: on the FP8 path P_ij = E4M3FN(fl32(p_ij * 448)),
 *           P's static scale 448 putting p in [0, 1] at the top of the
 *           format's range; on the FP16 path P_ij = fl16(p_ij) (bf16 for bf16
 *           inputs) ([guide] sec. 1: V in FP8 or FP16);
 *   sums    acc_c = sum_j P_ij V_jc and l = sum_j P_ij over the same rounded
 *           P, in fp64: the normaliser sums the weights that multiply V, so
 *           the normalised weights P_ij / l of a row sum to one and every
 *           output is a convex combination of the rows of V;
 *   output  out_ic = acc_c * vscale_c / l + vmean_c (FP8 path; P's scale
 *           cancels between acc and l) or acc_c / l + vmean_c (FP16 path)
 *           ([guide] sec. 4.2: smooth_v adds back the mean it subtracted);
 *   lse     (m - log2(Pscale) + log2 l) ln 2, plus sm_scale * sum_c q8_ic
 *           qscale_i kmean_c when K was smoothed, so that it is the
 *           log-sum-exp of the unsmoothed scores ([guide] sec. 4.1:
 *           return_lse); Pscale is 448 on the FP8 path and 1 otherwise.
 *
 * Causal masking keeps keys j <= i + causal_shift (top-left alignment when the
 * shift is 0); keys j >= nk do not exist.  Tiles with no visible key are
 * skipped.
 *
 * Rounding sensitivity ("allowance").  Another evaluation of the same steps
 * may form the exponent with a different rounding order; if its value of P_ij
 * before the operand rounding lies within a factor 2^(+-delta_ij) of this
 * one, with
 *     delta_ij = band_f * f_ij + band_x * (|s_ij| + |m'| + 8),
 *     f_ij = c_i * kscale_j (one integer score unit, in log2 units),
 * its operand can differ from P_ij only where the interval
 * [P 2^-delta, P 2^delta] contains a rounding boundary of the operand format.
 * Changing the operands of a row by dP_j moves its output by
 * sum_j dP_j (V_jc - out_c) / (l + sum_j dP_j), so for every such key the
 * width of the operand interval is recorded, and `allow` (if not NULL)
 * receives  sum_j |dP_j| |V_jc - out_c| / (l - sum_j |dP_j|)  in output units
 * (each dP_j carried to the final reference maximum like acc), and
 * `lse_allow` (if not NULL) receives -ln(1 - sum_j |dP_j| / l), the most
 * those changes can move ln l and so the log-sum-exp.  With
 * band_f = band_x = 0 both allowances are 0.
 *
 * q8: nq x dp; qscale: nq (per row, expanded from its group); k8: nk x dp;
 * kscale: nk (per key, expanded); vval: nk x dp values of the PV operand
 * (decoded E4M3 codes on the FP8 path, fp16/bf16 values on the FP16 path);
 * vscale: dp (FP8 path) or NULL; vmean, kmean: dp or NULL.
 * p_mode: 0 FP8, 1 fp16, 2 bf16.
 * rows: nrows query indices to compute; out: nrows x dp; lse: nrows or NULL;
 * sdump: nrows x nk int32 scores or NULL; allow: nrows x dp or NULL;
 * lse_pq: nrows or NULL, the part of lse that comes from rounding P to its
 * operand format: |ln(sum of rounded P) - ln(sum of unrounded P)|;
 * pdump: nrows x nk or NULL, the operand value P_ij of each key at its own
 * tile's reference maximum (0 for keys the row does not see); mdump:
 * nrows x nk or NULL, that reference maximum m' (-inf for unseen keys);
 * lse_allow: nrows or NULL (see above).                                       */
static double p_operand(double p, int p_mode) {
    if (p_mode == 0) return e4m3_value(p < E4M3_MAX ? p : E4M3_MAX);
    return fmt_rne(p, p_mode == 2 ? 7 : 10, p_mode == 2 ? -126 : -14);
}

int oracle_attn_rows(int nq, int nk, int dp,
                     const int8_t* q8, const float* qscale,
                     const int8_t* k8, const float* kscale,
                     const float* vval, const float* vscale, const float* vmean,
                     const float* kmean, float sm_scale, int causal, int causal_shift,
                     int bk, int p_mode, double band_f, double band_x,
                     int nrows, const int32_t* rows,
                     double* out, double* lse, int32_t* sdump, double* allow, double* lse_pq,
                     double* pdump, float* mdump, double* lse_allow) {
    if (bk <= 0 || dp <= 0 || nk <= 0) return -1;
    const float LOG2E = 1.4426950408889634f;
    const double pscale = p_mode == 0 ? E4M3_MAX : 1.0;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int ri = 0; ri < nrows; ++ri) {
        int i = rows[ri];
        if (i < 0 || i >= nq) { err = -2; continue; }
        int32_t* S = (int32_t*)malloc(sizeof(int32_t) * (size_t)nk);
        float* s = (float*)malloc(sizeof(float) * (size_t)nk);
        double* acc = (double*)calloc((size_t)dp, sizeof(double));
        int* fj = (int*)malloc(sizeof(int) * (size_t)nk);           /* keys whose operand may differ */
        double* fd = (double*)malloc(sizeof(double) * (size_t)nk);  /* their operand interval widths */
        float* fm = (float*)malloc(sizeof(float) * (size_t)nk);     /* their tile's reference maximum */
        int nflip = 0;
        const int8_t* qi = q8 + (size_t)i * dp;
        for (int j = 0; j < nk; ++j) {
            int64_t dot = 0;
            const int8_t* kj = k8 + (size_t)j * dp;
            for (int c = 0; c < dp; ++c) dot += (int64_t)qi[c] * (int64_t)kj[c];
            S[j] = (int32_t)dot;
        }
        if (sdump) memcpy(sdump + (size_t)ri * nk, S, sizeof(int32_t) * (size_t)nk);
        volatile float ci = qscale[i] * sm_scale;
        volatile float ci2 = ci * LOG2E;
        for (int j = 0; j < nk; ++j) {
            volatile float t = (float)S[j] * kscale[j];              /* fp32 products, one rounding each */
            volatile float sj = t * ci2;
            s[j] = sj;
        }
        int last = nk - 1;
        if (causal) {
            long lim = (long)i + causal_shift;
            if (lim < last) last = (int)lim;
        }
        if (pdump)
            for (int j = 0; j < nk; ++j) pdump[(size_t)ri * nk + j] = 0.0;
        if (mdump)
            for (int j = 0; j < nk; ++j) mdump[(size_t)ri * nk + j] = -INFINITY;
        float m = -INFINITY;
        double l = 0.0, lu = 0.0;                          /* sums of rounded / unrounded P */
        for (int t0 = 0; t0 <= last; t0 += bk) {
            int t1 = t0 + bk - 1;
            if (t1 > last) t1 = last;
            float mt = -INFINITY;
            for (int j = t0; j <= t1; ++j) if (s[j] > mt) mt = s[j];
            float mn = mt > m ? mt : m;                     /* m' = max(m, tile maximum) */
            if (mn > m && m != -INFINITY) {
                double alpha = exp2((double)m - (double)mn);
                l *= alpha;
                lu *= alpha;
                for (int c = 0; c < dp; ++c) acc[c] *= alpha;
            }
            m = mn;
            for (int j = t0; j <= t1; ++j) {
                volatile float x = s[j] - m;                 /* fp32 subtraction, x <= 0 */
                float p = (float)exp2((double)x);            /* fp64 exp2 rounded to fp32 */
                volatile float pp = (float)((double)p * pscale);   /* fl32(p * Pscale); exact when Pscale = 1 */
                double pq = p_operand(pp, p_mode);
                l += pq;
                lu += (double)pp;
                const float* vj = vval + (size_t)j * dp;
                for (int c = 0; c < dp; ++c) acc[c] += pq * (double)vj[c];
                if (pdump) pdump[(size_t)ri * nk + j] = pq;
                if (mdump) mdump[(size_t)ri * nk + j] = m;
                double delta = band_f * (double)ci2 * (double)kscale[j] +
                               band_x * (fabs((double)s[j]) + fabs((double)m) + 8.0);
                if (delta > 0.0) {
                    double lo = p_operand((double)pp * exp2(-delta), p_mode);
                    double hi = p_operand((double)pp * exp2(delta), p_mode);
                    if (hi > lo) { fj[nflip] = j; fd[nflip] = hi - lo; fm[nflip] = m; ++nflip; }
                }
            }
        }
        double sum_dp = 0.0;                               /* interval widths at the final reference */
        for (int k = 0; k < nflip; ++k) {
            fd[k] *= exp2((double)fm[k] - (double)m);
            sum_dp += fd[k];
        }
        for (int c = 0; c < dp; ++c) {
            double sc = p_mode == 0 ? (double)vscale[c] : 1.0;
            double o = acc[c] / l;                          /* operand units */
            out[(size_t)ri * dp + c] = o * sc + (vmean ? (double)vmean[c] : 0.0);
            if (allow) {
                double a = 0.0;
                for (int k = 0; k < nflip; ++k) a += fd[k] * fabs((double)vval[(size_t)fj[k] * dp + c] - o);
                double den = l - sum_dp;
                allow[(size_t)ri * dp + c] = nflip == 0 ? 0.0 : (den > 0.0 ? a * sc / den : INFINITY);
            }
        }
        if (lse) {
            double corr = 0.0;
            if (kmean) {
                for (int c = 0; c < dp; ++c) corr += (double)qi[c] * (double)qscale[i] * (double)kmean[c];
                corr *= (double)sm_scale;
            }
            lse[ri] = ((double)m - log2(pscale) + log2(l)) * M_LN2 + corr;
        }
        if (lse_pq) lse_pq[ri] = l > 0.0 ? fabs(log(l) - log(lu)) : 0.0;
        if (lse_allow) lse_allow[ri] = sum_dp <= 0.0 ? 0.0 : (sum_dp < l ? -log1p(-sum_dp / l) : INFINITY);
        free(S); free(s); free(acc); free(fj); free(fd); free(fm);
    }
    return err;
}

/* ------------------------------------------------------------------------ */
/* Exact attention in fp64 (no quantization), for selected rows:
 * out_i = sum_j softmax_j(sm_scale q_i.k_j) v_j, lse_i = log sum_j exp(...).
 * Same causal convention as above.  q: nq x d, k, v: nk x d (fp64).          */
int oracle_attn_exact(int nq, int nk, int d, const double* q, const double* k, const double* v,
                      double sm_scale, int causal, int causal_shift,
                      int nrows, const int32_t* rows, double* out, double* lse) {
    int err = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int ri = 0; ri < nrows; ++ri) {
        int i = rows[ri];
        if (i < 0 || i >= nq) { err = -2; continue; }
        int last = nk - 1;
        if (causal) {
            long lim = (long)i + causal_shift;
            if (lim < last) last = (int)lim;
        }
        double* s = (double*)malloc(sizeof(double) * (size_t)nk);
        double mx = -INFINITY;
        for (int j = 0; j <= last; ++j) {
            double dot = 0.0;
            for (int c = 0; c < d; ++c) dot += q[(size_t)i * d + c] * k[(size_t)j * d + c];
            s[j] = dot * sm_scale;
            if (s[j] > mx) mx = s[j];
        }
        double l = 0.0;
        for (int j = 0; j <= last; ++j) { s[j] = exp(s[j] - mx); l += s[j]; }
        for (int c = 0; c < d; ++c) {
            double o = 0.0;
            for (int j = 0; j <= last; ++j) o += s[j] * v[(size_t)j * d + c];
            out[(size_t)ri * d + c] = o / l;
        }
        if (lse) lse[ri] = mx + log(l);
        free(s);
    }
    return err;
}
