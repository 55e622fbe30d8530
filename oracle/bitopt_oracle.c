/*
 * bitopt_oracle.c -- plain, slow CPU oracle of the 8-bit block-wise optimizer step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header, table or constant generator with the HIP
 * library; the two meet only through caller-owned data (codebooks, codes, absmax,
 * parameters) handed to both.
 *
 * Sources (page titles and sections):
 *   [P1] "[XPU] Implemented 8bit optimizers in triton #1692" -- benchmark/test script
 *        (optimizer table, state-name table, dequantize_blockwise call).
 *   [P2] bitsandbytes "optim_overview" -- Optimizer2State / Optimizer1State
 *        hyper-parameter lists (lr, betas, eps, weight_decay, min_8bit_size,
 *        max_unorm, skip_zeros, alpha, t_alpha, t_beta3).
 *   [P3] "Support skip_zeros in the XPU Triton optimizer kernels #2097" --
 *        description, Implementation and Tests sections.
 *   [P4] "8-bit Optimizers via Block-wise Quantization" -- abstract (block-wise
 *        dynamic quantization) and the citing-papers quote from the k-bit scaling
 *        laws paper (dynamic exponent data type).
 *
 * Arithmetic precision.  Optimizer state values live in fp32 between decode and
 * encode, as in the 32-bit optimizers [P1] compares against; every element
 * operation below is one IEEE fp32 operation in the order written (compile with
 * -ffp-contract=off, no fast-math).  Per-step scalars are formed in double from the
 * fp32 hyper-parameters and rounded once to fp32.  The nearest-code decision is
 * taken on fp32 distances, the precision the device takes it in.
 *
 * Structure.  Every routine loops over quantization blocks, then over elements in
 * index order.  OpenMP, when enabled, only splits the block loop; blocks are
 * independent, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OREF_EXPORT __attribute__((visibility("default")))

enum { OREF_F32 = 0, OREF_F16 = 1, OREF_BF16 = 2 };
enum { OREF_ADAM = 0, OREF_ADEMAMIX = 1, OREF_MOMENTUM = 2, OREF_LION = 3, OREF_RMSPROP = 4, OREF_ADAGRAD = 5 };
enum { OREF_MAXB = 4096 };

/* Hyper-parameters of one step call; field meanings follow [P2] Optimizer2State /
 * Optimizer1State.  t_alpha / t_beta3 <= 0 mean "None".  max_unorm == 0 means off. */
typedef struct {
    int32_t optimizer;
    float lr, beta1, beta2, beta3, eps, weight_decay, alpha;
    int32_t t_alpha, t_beta3;
    float max_unorm;
    int32_t skip_zeros;
    int32_t blocksize;
} oref_hparams;

/* ------------------------------------------------------------------------- */
/* Number formats.  fp16/bf16 -> fp32 is exact; fp32 -> fp16/bf16 rounds to     */
/* nearest, ties to even, overflow to infinity (IEEE 754 default rounding).     */
/* ------------------------------------------------------------------------- */

static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static float half_to_float(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    int exp = (h >> 10) & 0x1f;
    uint32_t man = h & 0x3ff;
    if (exp == 0x1f)                       /* inf / nan */
        return u2f(sign | 0x7f800000u | (man << 13));
    if (exp == 0) {                        /* zero / subnormal: man * 2^-24 */
        float v = (float)man * 5.9604644775390625e-08f;
        return sign ? -v : v;
    }
    return u2f(sign | ((uint32_t)(exp - 15 + 127) << 23) | (man << 13));
}

static uint16_t float_to_half(float f)
{
    uint32_t u = f2u(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
    uint32_t a = u & 0x7fffffffu;
    if (a >= 0x7f800000u)                  /* inf or nan */
        return (uint16_t)(sign | 0x7c00 | (a > 0x7f800000u ? 0x200 : 0));
    /* Scale to an integer count of the target's least significant unit and round
     * that integer to nearest-even. */
    int e = (int)(a >> 23) - 127;          /* unbiased exponent */
    if (e >= 16) return (uint16_t)(sign | 0x7c00);
    uint32_t m = (a & 0x7fffff) | (e > -127 ? 0x800000u : 0); /* 24-bit significand */
    if (e == -127) e = -126;               /* fp32 subnormal */
    /* value = m * 2^(e-23).  Half unit: 2^(max(e,-14)-10). */
    int unit_exp = (e < -14 ? -14 : e) - 10;
    int shift = unit_exp - (e - 23);        /* bits of m below the target unit */
    uint32_t q;
    if (shift >= 32) {
        q = 0;
    } else if (shift <= 0) {
        q = m << (-shift);
    } else {
        uint32_t rem = m & ((1u << shift) - 1);
        uint32_t halfway = 1u << (shift - 1);
        q = m >> shift;
        if (rem > halfway || (rem == halfway && (q & 1))) q++;
    }
    /* q counts units of 2^unit_exp.  Re-assemble. */
    if (unit_exp == -24)                   /* units of 2^-24: the bit pattern is q itself */
        return (uint16_t)(sign | q);        /* (q == 0x400 is the smallest normal, 0x800 is 2^-13) */
    /* normal: q in [2^10, 2^11]; q == 2^11 means carry into the exponent */
    int he = unit_exp + 10 + 15;
    if (q >= 0x800) { q >>= 1; he++; }
    if (he >= 31) return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (he << 10) | (q & 0x3ff));
}

static float bf16_to_float(uint16_t b) { return u2f((uint32_t)b << 16); }

static uint16_t float_to_bf16(float f)
{
    uint32_t u = f2u(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40); /* quiet nan */
    uint32_t lsb = (u >> 16) & 1;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

static float load_elem(const void* base, int dtype, int64_t i)
{
    if (dtype == OREF_F32) return ((const float*)base)[i];
    if (dtype == OREF_F16) return half_to_float(((const uint16_t*)base)[i]);
    return bf16_to_float(((const uint16_t*)base)[i]);
}

static void store_elem(void* base, int dtype, int64_t i, float v)
{
    if (dtype == OREF_F32) ((float*)base)[i] = v;
    else if (dtype == OREF_F16) ((uint16_t*)base)[i] = float_to_half(v);
    else ((uint16_t*)base)[i] = float_to_bf16(v);
}

OREF_EXPORT void oref_round_to_dtype(const float* x, int64_t n, int dtype, void* out)
{
    for (int64_t i = 0; i < n; i++) store_elem(out, dtype, i, x[i]);
}

OREF_EXPORT void oref_widen_from_dtype(const void* x, int64_t n, int dtype, float* out)
{
    for (int64_t i = 0; i < n; i++) out[i] = load_elem(x, dtype, i);
}

/* ------------------------------------------------------------------------- */
/* Dynamic-exponent codebook [P4, citing-papers quote; abstract].               */
/*                                                                               */
/* An 8-bit pattern is read as: (signed map) one sign bit, then a run of E zero  */
/* bits giving the base-10 exponent 10^-E, then a 1 indicator bit, then the      */
/* remaining k bits as a linear fraction.  The fraction bits cut the decade      */
/* [0.1, 1] * 10^-E into 2^k equal bins; a pattern stands for its bin's midpoint.*/
/* The unsigned map has no sign bit, so every decade has one more fraction bit.  */
/* The patterns with no indicator bit left (all zero, and in the signed map its  */
/* negative twin) are given the values 0 and +1.0, so that a block's absmax      */
/* itself is representable exactly.  Values are formed in double, rounded once   */
/* to fp32 and sorted ascending; a code is its rank in the sorted array.         */
/* ------------------------------------------------------------------------- */

static double decode_pattern(int is_signed, unsigned pattern)
{
    int nbits = is_signed ? 7 : 8;          /* bits after the sign bit */
    unsigned body = is_signed ? (pattern & 0x7f) : (pattern & 0xff);
    double sgn = (is_signed && (pattern & 0x80)) ? -1.0 : 1.0;
    int zeros = 0;
    while (zeros < nbits && !(body & (1u << (nbits - 1 - zeros)))) zeros++;
    int k = nbits - 1 - zeros;              /* fraction bits after the indicator */
    /* Patterns whose indicator would sit past the last decade that keeps a
     * fraction field: signed -> body 0 (two patterns: 0 and +1.0);
     * unsigned -> body 0 (0.0) and body 1 (+1.0). */
    if (is_signed) {
        if (body == 0) return (pattern & 0x80) ? 1.0 : 0.0;
    } else {
        if (body == 0) return 0.0;
        if (body == 1) return 1.0;
    }
    unsigned frac = body & ((1u << k) - 1u);
    double decade = pow(10.0, -(double)zeros);
    double bins = (double)(1u << k);
    double mid = 0.1 + 0.9 * ((double)frac + 0.5) / bins;
    return sgn * decade * mid;
}

static int cmp_float(const void* a, const void* b)
{
    float x = *(const float*)a, y = *(const float*)b;
    return (x > y) - (x < y);
}

OREF_EXPORT int oref_dynamic_map(int is_signed, float* out)
{
    for (unsigned pat = 0; pat < 256; pat++)
        out[pat] = (float)decode_pattern(is_signed, pat);
    qsort(out, 256, sizeof(float), cmp_float);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Block-wise codec [P1 test body: dequantize_blockwise(code, absmax, A,        */
/* blocksize); P4 abstract: independent blocks].                                 */
/* ------------------------------------------------------------------------- */

/* The plain definition of "nearest codebook entry": the index j minimising the
 * fp32 distance |x - Q[j]|; on an exact tie the smaller index wins.  The pages say
 * nothing about non-finite data; the reading here: a NaN value (it arises only
 * from a NaN state, or from an infinite state in a block whose absmax is then
 * infinite and whose reciprocal is 0) has no nearest entry and is encoded as +0
 * is, so a poisoned element decodes to zero instead of an arbitrary code. */
static int nearest_code(const float* Q, float x)
{
    if (x != x) x = 0.0f;
    int best = 0;
    float bd = fabsf(x - Q[0]);
    for (int j = 1; j < 256; j++) {
        float d = fabsf(x - Q[j]);
        if (d < bd) { bd = d; best = j; }
    }
    return best;
}

OREF_EXPORT void oref_nearest(const float* Q, const float* x, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)nearest_code(Q, x[i]);
}

/* Encode one block of fp32 values: absmax A = max |s| over the values that are
 * not NaN (exact; 0 when there are none -- a NaN never becomes the scale), one correctly
 * rounded reciprocal r = 1/A per block (r = 0 when A = 0), then the nearest code
 * of s*r.  A subnormal A can have a reciprocal beyond the fp32 range; such a block
 * is first scaled by 2^24 (exact): r = 1/(A*2^24) and the values (s*2^24)*r.
 * Wherever 1/A is finite this gives the same bits as the plain form (a power of
 * two commutes with rounding in the normal range), so the normalization stays
 * invariant under power-of-two scaling of the block. */
static float encode_block(const float* s, int len, const float* Q, uint8_t* codes)
{
    float A = 0.0f;
    for (int i = 0; i < len; i++) {
        float a = fabsf(s[i]);
        if (a > A) A = a;
    }
    float c = (A < 0x1p-126f) ? 0x1p24f : 1.0f;
    float r = (A == 0.0f) ? 0.0f : 1.0f / (A * c);
    for (int i = 0; i < len; i++) {
        float x = (s[i] * c) * r;
        codes[i] = (uint8_t)nearest_code(Q, x);
    }
    return A;
}

OREF_EXPORT int oref_quantize_blockwise(const void* x, int dtype, int64_t n, const float* qmap,
                                        int32_t blocksize, uint8_t* codes, float* absmax)
{
    if (n < 0 || blocksize < 1 || blocksize > OREF_MAXB) return -1;
    int64_t nb = (n + blocksize - 1) / blocksize;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; b++) {
        float s[OREF_MAXB];
        int64_t off = b * blocksize;
        int len = (int)((n - off) < blocksize ? (n - off) : blocksize);
        for (int i = 0; i < len; i++) s[i] = load_elem(x, dtype, off + i);
        absmax[b] = encode_block(s, len, qmap, codes + off);
    }
    return 0;
}

OREF_EXPORT int oref_dequantize_blockwise(const uint8_t* codes, const float* absmax, const float* qmap,
                                          int64_t n, int32_t blocksize, void* out, int dtype)
{
    if (n < 0 || blocksize < 1) return -1;
    for (int64_t i = 0; i < n; i++) {
        float v = qmap[codes[i]] * absmax[i / blocksize];
        store_elem(out, dtype, i, v);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Per-step scalars.  Formed in double from the fp32 hyper-parameters, rounded   */
/* once to fp32.  Step t is 1-based.                                             */
/*   ic1 = 1/(1-beta1^t), rs2 = 1/sqrt(1-beta2^t)  (Adam bias corrections)       */
/*   decay = 1 - lr*wd                              (decoupled weight decay)      */
/*   AdEMAMix [P2: alpha, t_alpha, t_beta3]: alpha(t) ramps linearly to alpha    */
/*   over t_alpha steps; beta3(t) moves the slow EMA's half-life linearly from   */
/*   beta1's to beta3's over t_beta3 steps, capped at beta3.                     */
/* ------------------------------------------------------------------------- */

typedef struct {
    float lr, b1, b2, eps, wd;
    float omb1, omb2, ic1, rs2, decay;
    float b3t, omb3, alpha_t;
} step_scalars;

OREF_EXPORT double oref_beta3_schedule(double beta1, double beta3, int32_t t, int32_t T)
{
    if (T <= 0) return beta3;
    double lb1 = log(beta1), lb3 = log(beta3);
    double f = (double)t / (double)T;
    double v = exp(lb1 * lb3 / ((1.0 - f) * lb3 + f * lb1));
    return v < beta3 ? v : beta3;
}

OREF_EXPORT double oref_alpha_schedule(double alpha, int32_t t, int32_t T)
{
    if (T <= 0) return alpha;
    double f = (double)t / (double)T;
    return alpha * (f < 1.0 ? f : 1.0);
}

static void make_scalars(const oref_hparams* h, int32_t t, step_scalars* s)
{
    double b1 = h->beta1, b2 = h->beta2;
    s->lr = h->lr; s->b1 = h->beta1; s->b2 = h->beta2; s->eps = h->eps; s->wd = h->weight_decay;
    s->omb1 = (float)(1.0 - b1);
    s->omb2 = (float)(1.0 - b2);
    s->ic1 = (float)(1.0 / (1.0 - pow(b1, (double)t)));
    s->rs2 = (float)(1.0 / sqrt(1.0 - pow(b2, (double)t)));
    s->decay = (float)(1.0 - (double)h->lr * (double)h->weight_decay);
    double b3t = oref_beta3_schedule(b1, (double)h->beta3, t, h->t_beta3);
    s->b3t = (float)b3t;
    s->omb3 = (float)(1.0 - b3t);
    s->alpha_t = (float)oref_alpha_schedule((double)h->alpha, t, h->t_alpha);
}

OREF_EXPORT void oref_step_scalars(const oref_hparams* h, int32_t t, float* out13)
{
    step_scalars s;
    make_scalars(h, t, &s);
    float v[13] = {s.lr, s.b1, s.b2, s.eps, s.wd, s.omb1, s.omb2, s.ic1, s.rs2, s.decay,
                   s.b3t, s.omb3, s.alpha_t};
    memcpy(out13, v, sizeof(v));
}

/* ------------------------------------------------------------------------- */
/* The step.  One routine serves the 8-bit block-wise mode (states decoded from  */
/* codes and re-encoded) and the 32-bit mode (the codec is the identity on fp32  */
/* states).                                                                      */
/*                                                                               */
/* State slots per optimizer ([P1] state-name table):                            */
/*   Adam/AdamW : s1 = exp_avg m (signed map), s2 = exp_avg_sq v (unsigned map)  */
/*   AdEMAMix   : s1 = m1 then m2 stacked (signed map, shared; absmax stacked),   */
/*                s2 = nu (unsigned map)                                         */
/*   Momentum   : s1 = momentum_buffer (signed map)                              */
/*   Lion       : s1 = exp_avg (signed map)                                      */
/*   RMSprop    : s1 = square_avg (non-negative: the unsigned map)               */
/*   Adagrad    : s1 = sum of squared gradients (unsigned map)                   */
/* (the maps are the caller's; these are the ones the tests hand in)              */
/* ------------------------------------------------------------------------- */

typedef struct {
    int quantized;            /* 1: uint8 codes + absmax; 0: fp32 state arrays */
    void* s1;                 /* uint8* or float*; AdEMAMix holds 2n entries */
    void* s2;
    float* absmax1;           /* AdEMAMix holds 2*nb entries */
    float* absmax2;
    const float* q1;
    const float* q2;
} state_io;

static int num_states(int opt) { return opt == OREF_ADEMAMIX ? 3 : (opt <= OREF_ADEMAMIX ? 2 : 1); }

/* Which slot (array, offset in elements, absmax offset in blocks, map) state k of
 * optimizer opt lives in. */
static void slot_of(int opt, int k, int64_t n, int64_t nb, const state_io* io,
                    void** arr, int64_t* eoff, float** am, int64_t* aoff, const float** q)
{
    *eoff = 0; *aoff = 0;
    if (k == 0) { *arr = io->s1; *am = io->absmax1; *q = io->q1; }
    else if (opt == OREF_ADEMAMIX && k == 1) { *arr = io->s1; *am = io->absmax1; *q = io->q1; *eoff = n; *aoff = nb; }
    else { *arr = io->s2; *am = io->absmax2; *q = io->q2; }
}

static float sign_of(float c) { return c > 0.0f ? 1.0f : (c < 0.0f ? -1.0f : 0.0f); }

static void step_block(const oref_hparams* h, const step_scalars* sc, int64_t b, int64_t n, int B,
                       void* p, const void* g, int dtype, const state_io* io)
{
    const int opt = h->optimizer;
    const int ns = num_states(opt);
    const int64_t nb = (n + B - 1) / B;
    const int64_t off = b * (int64_t)B;
    const int len = (int)((n - off) < B ? (n - off) : B);

    /* Blocks up to OREF_MAXB elements live on the stack; a tensor-wide block
     * (blocksize 0: the whole tensor) on the heap. */
    float pv_s[OREF_MAXB], gv_s[OREF_MAXB], dv_s[OREF_MAXB], st_s[3][OREF_MAXB];
    int skip_s[OREF_MAXB];
    float *pv = pv_s, *gv = gv_s, *dv = dv_s, *st[3] = {st_s[0], st_s[1], st_s[2]};
    int* skip = skip_s;
    float* heap = NULL;
    int* heap_skip = NULL;
    if (len > OREF_MAXB) {
        heap = (float*)malloc(sizeof(float) * (size_t)len * 6);
        heap_skip = (int*)malloc(sizeof(int) * (size_t)len);
        if (!heap || !heap_skip) { free(heap); free(heap_skip); return; }
        pv = heap; gv = heap + len; dv = heap + 2 * (size_t)len;
        st[0] = heap + 3 * (size_t)len; st[1] = heap + 4 * (size_t)len; st[2] = heap + 5 * (size_t)len;
        skip = heap_skip;
    }

    void* arr[3]; int64_t eoff[3]; float* am[3]; int64_t aoff[3]; const float* q[3];
    for (int k = 0; k < ns; k++) slot_of(opt, k, n, nb, io, &arr[k], &eoff[k], &am[k], &aoff[k], &q[k]);

    /* Load parameters, gradients and the decoded states. */
    int any_live = 0;
    for (int i = 0; i < len; i++) {
        pv[i] = load_elem(p, dtype, off + i);
        gv[i] = load_elem(g, dtype, off + i);
        skip[i] = h->skip_zeros && (gv[i] == 0.0f);   /* raw gradient, before decay [P3] */
        if (!skip[i]) any_live = 1;
        for (int k = 0; k < ns; k++) {
            if (io->quantized) {
                uint8_t c = ((const uint8_t*)arr[k])[eoff[k] + off + i];
                st[k][i] = q[k][c] * am[k][aoff[k] + b];
            } else {
                st[k][i] = ((const float*)arr[k])[eoff[k] + off + i];
            }
        }
    }
    /* A block whose every gradient is zero is left completely untouched [P3]. */
    if (h->skip_zeros && !any_live) { free(heap); free(heap_skip); return; }

    /* Element updates: new states in st, parameter step in dv. */
    for (int i = 0; i < len; i++) {
        if (skip[i]) { dv[i] = 0.0f; continue; }
        float gi = gv[i], pi = pv[i];
        float t1, t2;
        switch (opt) {
        case OREF_ADAM: {
            float m = st[0][i], v = st[1][i];
            t1 = sc->b1 * m; t2 = sc->omb1 * gi; m = t1 + t2;
            float gg = gi * gi;
            t1 = sc->b2 * v; t2 = sc->omb2 * gg; v = t1 + t2;
            float d = sqrtf(v) * sc->rs2;
            d = d + sc->eps;
            float mh = m * sc->ic1;
            float u = mh / d;
            dv[i] = sc->lr * u;
            st[0][i] = m; st[1][i] = v;
            break;
        }
        case OREF_ADEMAMIX: {
            float m1 = st[0][i], m2 = st[1][i], nu = st[2][i];
            t1 = sc->b1 * m1; t2 = sc->omb1 * gi; m1 = t1 + t2;
            t1 = sc->b3t * m2; t2 = sc->omb3 * gi; m2 = t1 + t2;
            float gg = gi * gi;
            t1 = sc->b2 * nu; t2 = sc->omb2 * gg; nu = t1 + t2;
            float d = sqrtf(nu) * sc->rs2;
            d = d + sc->eps;
            t1 = m1 * sc->ic1; t2 = sc->alpha_t * m2;
            float num = t1 + t2;
            float u = num / d;
            dv[i] = sc->lr * u;
            st[0][i] = m1; st[1][i] = m2; st[2][i] = nu;
            break;
        }
        case OREF_MOMENTUM: {
            float buf = st[0][i];
            t1 = sc->wd * pi; float g2 = gi + t1;          /* decay folded into the gradient */
            t1 = sc->b1 * buf; buf = t1 + g2;
            dv[i] = sc->lr * buf;
            st[0][i] = buf;
            break;
        }
        case OREF_RMSPROP: {
            /* [P1] optimizer table: RMSprop8bit(p, 0.01, 0.9) against torch.optim.RMSprop
             * (lr 0.01, alpha 0.9): square_avg = alpha*square_avg + (1-alpha)*g'^2,
             * p -= lr * g'/(sqrt(square_avg) + eps), g' = g + wd*p (decay folded in). */
            float v = st[0][i];
            t1 = sc->wd * pi; float g2 = gi + t1;
            float gg = g2 * g2;
            t1 = sc->b1 * v; t2 = sc->omb1 * gg; v = t1 + t2;
            float d = sqrtf(v);
            d = d + sc->eps;
            float u = g2 / d;
            dv[i] = sc->lr * u;
            st[0][i] = v;
            break;
        }
        case OREF_ADAGRAD: {
            /* [P2]: the 1-state example.  torch.optim.Adagrad (no lr decay, zero initial
             * accumulator): sum += g'^2, p -= lr * g'/(sqrt(sum) + eps), g' = g + wd*p. */
            float v = st[0][i];
            t1 = sc->wd * pi; float g2 = gi + t1;
            float gg = g2 * g2;
            v = v + gg;
            float d = sqrtf(v);
            d = d + sc->eps;
            float u = g2 / d;
            dv[i] = sc->lr * u;
            st[0][i] = v;
            break;
        }
        default: { /* Lion */
            float m = st[0][i];
            t1 = sc->b1 * m; t2 = sc->omb1 * gi;
            float c = t1 + t2;
            dv[i] = sc->lr * sign_of(c);
            t1 = sc->b2 * m; t2 = sc->omb2 * gi; m = t1 + t2;
            st[0][i] = m;
            break;
        }
        }
    }

    /* max_unorm [P2]: per block, the update norm is capped at max_unorm times the
     * block's parameter norm.  Squares in fp32, sums in double. */
    float clip = 1.0f;
    int clipped = 0;
    if (h->max_unorm > 0.0f) {
        double su = 0.0, sp = 0.0;
        for (int i = 0; i < len; i++) {
            if (!skip[i]) { float d2 = dv[i] * dv[i]; su += (double)d2; }
            float p2 = pv[i] * pv[i]; sp += (double)p2;
        }
        double U = sqrt(su), P = sqrt(sp);
        double lim = (double)h->max_unorm * P;
        if (U > lim) { clip = (float)(lim / U); clipped = 1; }
    }

    /* Parameter write-back (rounded to the parameter type); skipped elements keep
     * their exact previous bits. */
    for (int i = 0; i < len; i++) {
        if (skip[i]) continue;
        float d = dv[i];
        if (clipped) d = d * clip;
        float pn;
        if (opt == OREF_MOMENTUM || opt == OREF_RMSPROP || opt == OREF_ADAGRAD) pn = pv[i] - d;   /* coupled decay */
        else { float pd = pv[i] * sc->decay; pn = pd - d; }
        store_elem(p, dtype, off + i, pn);
    }

    /* Re-encode the states. */
    for (int k = 0; k < ns; k++) {
        if (io->quantized) {
            uint8_t* codes = (uint8_t*)arr[k] + eoff[k] + off;
            am[k][aoff[k] + b] = encode_block(st[k], len, q[k], codes);
        } else {
            float* dst = (float*)arr[k] + eoff[k] + off;
            for (int i = 0; i < len; i++) if (!skip[i]) dst[i] = st[k][i];
        }
    }
    free(heap);
    free(heap_skip);
}

static int check_hparams(const oref_hparams* h, int32_t step, int64_t n)
{
    if (!h || step < 1 || n < 0) return -1;
    if (h->optimizer < OREF_ADAM || h->optimizer > OREF_ADAGRAD) return -1;
    /* blocksize 0: one block spanning the tensor (non-block-wise 8-bit) */
    if (h->blocksize < 0 || h->blocksize > OREF_MAXB) return -1;
    if (h->blocksize == 0 && n > INT32_MAX) return -1;
    return 0;
}

static int run_step(const oref_hparams* h, int32_t step, void* p, const void* g, int dtype, int64_t n,
                    const state_io* io, const int64_t* blocks, int64_t nblocks)
{
    if (check_hparams(h, step, n)) return -1;
    step_scalars sc;
    make_scalars(h, step, &sc);
    if (n == 0) return 0;
    const int B = h->blocksize ? h->blocksize : (int)n;
    const int64_t nb = (n + B - 1) / B;
    if (blocks) {
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < nblocks; j++)
            if (blocks[j] >= 0 && blocks[j] < nb) step_block(h, &sc, blocks[j], n, B, p, g, dtype, io);
    } else {
#pragma omp parallel for schedule(static)
        for (int64_t b = 0; b < nb; b++) step_block(h, &sc, b, n, B, p, g, dtype, io);
    }
    return 0;
}

/* 8-bit block-wise step.  For 2-state optimizers (Adam/AdamW, AdEMAMix) pass
 * state2/absmax2/qmap2; for 1-state ones (Momentum, Lion) they are unused.
 * `blocks` (optional) restricts the step to the listed block indices. */
OREF_EXPORT int oref_step_8bit(const oref_hparams* h, int32_t step, void* p, const void* g, int dtype,
                               int64_t n, uint8_t* state1, uint8_t* state2, float* absmax1,
                               float* absmax2, const float* qmap1, const float* qmap2,
                               const int64_t* blocks, int64_t nblocks)
{
    state_io io = {1, state1, state2, absmax1, absmax2, qmap1, qmap2};
    return run_step(h, step, p, g, dtype, n, &io, blocks, nblocks);
}

/* 32-bit step: the same update with fp32 states and no codec (state1 holds m, or
 * m1 then m2 for AdEMAMix; state2 holds v / nu).  max_unorm blocks use blocksize. */
OREF_EXPORT int oref_step_32bit(const oref_hparams* h, int32_t step, void* p, const void* g, int dtype,
                                int64_t n, float* state1, float* state2,
                                const int64_t* blocks, int64_t nblocks)
{
    state_io io = {0, state1, state2, NULL, NULL, NULL, NULL};
    return run_step(h, step, p, g, dtype, n, &io, blocks, nblocks);
}

OREF_EXPORT void oref_set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

OREF_EXPORT int oref_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
