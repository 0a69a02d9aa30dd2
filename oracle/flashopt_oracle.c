/*
 * Oracle for the FlashAdamW and FlashSGD optimizer steps -- plain CPU C, one
 * element at a time, in the pages' order.  TEST INFRASTRUCTURE ONLY (see the header): the
 * product library neither links nor includes this file.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -fPIC -shared
 * (x86-64 SSE scalar float: every + - * / sqrt is one IEEE binary32 operation
 * rounded to nearest even; nearbyint() rounds half to even; no FTZ/DAZ).
 *
 * Readings of the pages that this file fixes (each is argued where it is used):
 *   R1  weight split (Alg. 1) -- not printed; ties away from zero, integer residual.
 *   R2  "round" in quantize() is torch.round: half to even.
 *   R3  the AdamW body follows the page's printed operation order exactly
 *       (bias corrections as divisions, then lr * mhat over sqrt(vhat) + eps).
 *   R12 non-finite values are out of contract; NaN is given code 0 / quiet
 *       NaN so that both sides of a parity test stay defined.
 *   R16 FlashSGD's update (given only as a bytes_per_param row) is
 *       torch.optim.SGD with momentum, in torch's order.
 */
#include "flashopt_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ bits */

static uint32_t bits_of(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float float_of(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* bf16 is the upper half of a binary32 pattern; widening is exact. */
static float bf16_to_f32(uint16_t b) { return float_of((uint32_t)b << 16); }

/* torch's float32 -> bfloat16 cast: round to nearest, ties to even (used only
 * when there is no master split: [SIM step()] then writes theta back cast to
 * the parameter's dtype). */
static uint16_t bf16_rne(float x)
{
    uint32_t u = bits_of(x);
    if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t hi = u >> 16, lo = u & 0xFFFFu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;
    return (uint16_t)hi;
}

/* -------------------------------------------------------- O0: binary16 */

/* binary16 has a 5-bit exponent (bias 15) and a 10-bit fraction: normal
 * values (1 + f/1024) 2^(E-15) for E = 1..30, subnormals f 2^-24, largest
 * finite 65504.  Rounding to nearest even is done on exactly scaled doubles. */
uint16_t oracle_f16_from_f32(float x)
{
    uint16_t sign = (uint16_t)((bits_of(x) >> 16) & 0x8000u);
    if (isnan(x)) return (uint16_t)(sign | 0x7E00u);
    if (isinf(x)) return (uint16_t)(sign | 0x7C00u);
    double a = fabs((double)x);
    if (a < 0x1p-14) {
        /* subnormal range: a multiple of 2^-24.  A result of 1024 steps is
         * the smallest normal, whose encoding is the same integer. */
        double k = nearbyint(a * 0x1p24);
        return (uint16_t)(sign | (uint16_t)k);
    }
    int e;
    double f = frexp(a, &e);            /* a = f 2^e, f in [0.5, 1) */
    int E = e - 1;                      /* a = (2f) 2^E, 2f in [1, 2) */
    double k = nearbyint(2.0 * f * 1024.0);   /* 11-bit significand, [1024, 2048] */
    if (k == 2048.0) { k = 1024.0; E += 1; }
    if (E > 15) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)(((E + 15) << 10) | ((int)k - 1024)));
}

void oracle_f16_array(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_from_f32(x[i]);
}

float oracle_f32_from_f16(uint16_t h)
{
    int neg = (h >> 15) & 1, E = (h >> 10) & 31, F = h & 1023;
    double v;
    if (E == 31) {
        if (F) return neg ? -NAN : NAN;
        v = INFINITY;
    } else if (E == 0) {
        v = ldexp((double)F, -24);
    } else {
        v = ldexp((double)(1024 + F), E - 25);
    }
    return (float)(neg ? -v : v);
}

/* ------------------------------------------------- O1/O2: weight split */

/* R1.  The pages call the split (S.compress / S.decompress in [SIM step()]
 * and [EQ eq_ecc()]) but do not print it.  What they fix: theta' is the bf16
 * rounding of the fp32 master ([EQ eq_ecc()] passes the bf16 cast of the master
 * to the correction-bit routine), rho is int8 for a 24-bit and int16 for a 32-bit
 * master ([SIM FlashAdamWSim.__init__]), and a bf16-exact parameter splits to
 * rho = 0 ([SIM step()], state init).  Reading:
 *   theta' = theta rounded to bf16, nearest, ties away from zero (on the
 *            magnitude); this is the only nearest rounding for which a 16-bit
 *            rho can hold every dropped residual, so the 32-bit master is
 *            lossless;
 *   D      = pattern(theta) - pattern(theta') * 2^16, in [-32768, 32767],
 *            i.e. the residual in units of theta's last binary32 place;
 *   rho    = D (32-bit master), or D/256 rounded half to even and clamped to
 *            [-128, 127] (24-bit master).
 * NaN keeps its upper half with the quiet bit set and rho = 0. */
static void split_one(float x, int master_bits, uint16_t *hi, int32_t *rho)
{
    uint32_t u = bits_of(x);
    if (isnan(x)) { *hi = (uint16_t)((u >> 16) | 0x0040u); *rho = 0; return; }
    uint32_t b = u >> 16;               /* truncated bf16 pattern, sign included */
    int32_t lo = (int32_t)(u & 0xFFFFu);
    int32_t D;
    if (lo >= 0x8000) {                 /* at or past the midpoint: magnitude rounds up */
        b += 1u;
        D = lo - 0x10000;
    } else {
        D = lo;
    }
    *hi = (uint16_t)b;
    if (master_bits == 32) {
        *rho = D;
    } else {
        double r = nearbyint((double)D / 256.0);
        if (r > 127.0) r = 127.0;
        if (r < -128.0) r = -128.0;
        *rho = (int32_t)r;
    }
}

int oracle_split(const float *x, int64_t n, int master_bits,
                 uint16_t *theta_bf16, void *rho)
{
    if (master_bits != 24 && master_bits != 32) return -1;
    for (int64_t i = 0; i < n; ++i) {
        int32_t r;
        split_one(x[i], master_bits, &theta_bf16[i], &r);
        if (master_bits == 32) ((int16_t *)rho)[i] = (int16_t)r;
        else ((int8_t *)rho)[i] = (int8_t)r;
    }
    return 0;
}

/* pattern(theta) = pattern(theta') * 2^16 + rho * 2^(16 - w), w = 8 or 16,
 * taken modulo 2^32 (a negative rho borrows from the bf16 half). */
static float reconstruct_one(uint16_t hi, int32_t rho, int master_bits)
{
    int64_t scale = (master_bits == 32) ? 1 : 256;
    int64_t v = ((int64_t)hi << 16) + (int64_t)rho * scale;
    return float_of((uint32_t)(v & 0xFFFFFFFFll));
}

int oracle_reconstruct(const uint16_t *theta_bf16, const void *rho, int64_t n,
                       int master_bits, float *x)
{
    if (master_bits != 24 && master_bits != 32) return -1;
    for (int64_t i = 0; i < n; ++i) {
        int32_t r = (master_bits == 32) ? ((const int16_t *)rho)[i]
                                        : ((const int8_t *)rho)[i];
        x[i] = reconstruct_one(theta_bf16[i], r, master_bits);
    }
    return 0;
}

/* ------------------------------------------------ O3/O4: group-32 codec */

#define GROUP 32   /* [QZ] module constant GROUP */

/* [QZ quantize()], Alg. 2 (momentum: signed + softsign) and Alg. 3
 * (variance: unsigned + sqrt) forward, one group of 32 at a time:
 *   the group is zero padded past n ([QZ _grouped()]);
 *   a_i = sqrt(x_i) if SQRT, else x_i;
 *   amax = max |a_i| (signed) or max a_i (unsigned);
 *   s = fp16(amax); d = 1 if s == 0 else float(s);
 *   y_i = a_i / d; with SOFTSIGN y_i = (2 y_i) / (1 + |y_i|);
 *   q_i = clamp(round(y_i * 127), -127, 127) or clamp(round(y_i * 255), 0, 255)
 * (R2: round half to even).  NaN codes are 0 (R12). */
int oracle_quantize(const float *x, int64_t n, unsigned spec,
                    void *codes, uint16_t *scales)
{
    const int is_signed = (spec & ORACLE_SIGNED) != 0;
    int64_t G = (n + GROUP - 1) / GROUP;
    for (int64_t g = 0; g < G; ++g) {
        float a[GROUP];
        for (int i = 0; i < GROUP; ++i) {
            int64_t k = g * GROUP + i;
            float v = (k < n) ? x[k] : 0.0f;
            if (spec & ORACLE_SQRT) v = sqrtf(v);
            a[i] = v;
        }
        float amax = is_signed ? fabsf(a[0]) : a[0];
        for (int i = 1; i < GROUP; ++i)
            amax = fmaxf(amax, is_signed ? fabsf(a[i]) : a[i]);
        uint16_t s = oracle_f16_from_f32(amax);
        scales[g] = s;
        float d = ((s & 0x7FFFu) == 0) ? 1.0f : oracle_f32_from_f16(s);
        for (int i = 0; i < GROUP; ++i) {
            int64_t k = g * GROUP + i;
            if (k >= n) break;
            float y = a[i] / d;
            if (spec & ORACLE_SOFTSIGN) {
                float num = 2.0f * y;
                float den = 1.0f + fabsf(y);
                y = num / den;
            }
            if (is_signed) {
                float r = nearbyintf(y * 127.0f);
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                ((int8_t *)codes)[k] = isnan(r) ? 0 : (int8_t)r;
            } else {
                float r = nearbyintf(y * 255.0f);
                if (r > 255.0f) r = 255.0f;
                if (r < 0.0f) r = 0.0f;
                ((uint8_t *)codes)[k] = isnan(r) ? 0 : (uint8_t)r;
            }
        }
    }
    return 0;
}

/* [QZ dequantize()], the inverse of Alg. 2/3:
 *   y = q / 127 (signed) or q / 255 (unsigned);
 *   with SOFTSIGN y = y / (2 - |y|);
 *   out = y * float(s); with SQRT out = out * out. */
int oracle_dequantize(const void *codes, const uint16_t *scales, int64_t n,
                      unsigned spec, float *out)
{
    const int is_signed = (spec & ORACLE_SIGNED) != 0;
    for (int64_t k = 0; k < n; ++k) {
        float s = oracle_f32_from_f16(scales[k / GROUP]);
        float q = is_signed ? (float)((const int8_t *)codes)[k]
                            : (float)((const uint8_t *)codes)[k];
        float y = q / (is_signed ? 127.0f : 255.0f);
        if (spec & ORACLE_SOFTSIGN) {
            float den = 2.0f - fabsf(y);
            y = y / den;
        }
        float o = y * s;
        if (spec & ORACLE_SQRT) o = o * o;
        out[k] = o;
    }
    return 0;
}

/* [QZ nmse()]: mean((orig - recon)^2) / mean(orig^2) in double, 0 when the
 * denominator is 0. */
double oracle_nmse(const float *orig, const float *recon, int64_t n)
{
    double den = 0.0, num = 0.0;
    for (int64_t i = 0; i < n; ++i) den += (double)orig[i] * (double)orig[i];
    if (n > 0) den /= (double)n;
    if (den == 0.0) return 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double e = (double)orig[i] - (double)recon[i];
        num += e * e;
    }
    return (num / (double)n) / den;
}

/* ------------------------------------------------------ O5: AdamW step */

typedef struct {
    float cwd, b1, c1, b2, c2, lr, eps, bc1, bc2;
} step_scalars;

/* Python floats are doubles; each scalar meets the float32 tensors rounded
 * once to float ([SIM step()]: `1 - lr * wd`, `1 - beta1`, `1 - beta1 ** t`,
 * `lr`, `eps`).  Python's float ** int is the C library's pow() on doubles. */
static void make_scalars(const oracle_hparams *h, step_scalars *s)
{
    double t = (double)h->step;
    s->cwd = (float)(1.0 - h->lr * h->weight_decay);
    s->b1 = (float)h->beta1;
    s->c1 = (float)(1.0 - h->beta1);
    s->b2 = (float)h->beta2;
    s->c2 = (float)(1.0 - h->beta2);
    s->lr = (float)h->lr;
    s->eps = (float)h->eps;
    s->bc1 = (float)(1.0 - pow(h->beta1, t));
    s->bc2 = (float)(1.0 - pow(h->beta2, t));
}

/* Body of Alg. 4 [SIM step()], "Standard AdamW update", decoupled weight
 * decay, torch convention, one float32 rounding per operation in the order
 * the page writes it (Python evaluates left to right):
 *   theta <- theta * (1 - lr wd)                 (skipped when wd = 0; R11:
 *                                                 a factor of 1.0 is exact)
 *   m     <- beta1 * m + (1 - beta1) * g
 *   v     <- beta2 * v + ((1 - beta2) * g) * g
 *   mhat  <- m / (1 - beta1^t)
 *   vhat  <- v / (1 - beta2^t)
 *   theta <- theta - (lr * mhat) / (sqrt(vhat) + eps) */
void oracle_adamw_update(float *theta, float *m, float *v, const float *g,
                         int64_t n, const oracle_hparams *h)
{
    step_scalars s;
    make_scalars(h, &s);
    for (int64_t i = 0; i < n; ++i) {
        float th = theta[i] * s.cwd;
        float m_decay = s.b1 * m[i];
        float m_new = s.c1 * g[i];
        float m1 = m_decay + m_new;
        float v_decay = s.b2 * v[i];
        float cg = s.c2 * g[i];
        float v_new = cg * g[i];
        float v1 = v_decay + v_new;
        float mhat = m1 / s.bc1;
        float vhat = v1 / s.bc2;
        float den = sqrtf(vhat) + s.eps;
        float step_num = s.lr * mhat;
        float upd = step_num / den;
        theta[i] = th - upd;
        m[i] = m1;
        v[i] = v1;
    }
}

static unsigned momentum_spec(int companded)
{
    return ORACLE_SIGNED | (companded ? ORACLE_SOFTSIGN : 0u);
}

static unsigned variance_spec(int companded)
{
    return companded ? ORACLE_SQRT : 0u;      /* unsigned, no softsign */
}

/* One step of [SIM step()] on one tensor: dequantize m and v, rebuild theta,
 * update, requantize m and v, re-split theta.  State init (zero codes and
 * scales, rho from splitting the bf16 parameter, i.e. rho = 0) is the
 * caller's; a zero-filled state reproduces it.
 * Which theta: `use_split = master_weight_bits is not None and p.dtype !=
 * torch.float32`.  With a split, theta = decompress(param, rho) and the
 * update is split again; without one and a bf16 parameter, theta is the bf16
 * value widened and the update is cast back with torch's bf16 cast (R14);
 * with an fp32 parameter (fp32_param), theta is the parameter itself, its
 * gradient is fp32, and the update is stored unchanged. */
int oracle_adamw_step(void *param, const void *grad, void *rho,
                      void *m_codes, uint16_t *m_scales,
                      void *v_codes, uint16_t *v_scales,
                      int64_t n, const oracle_hparams *h)
{
    if (n < 0 || h == NULL || h->step < 1) return -1;
    if (h->master_bits != 0 && h->master_bits != 24 && h->master_bits != 32) return -1;
    if (h->fp32_param && h->master_bits != 0) return -1;
    if (n == 0) return 0;
    size_t bytes = (size_t)n * sizeof(float);
    float *theta = (float *)malloc(bytes), *m = (float *)malloc(bytes);
    float *v = (float *)malloc(bytes), *g = (float *)malloc(bytes);
    if (!theta || !m || !v || !g) { free(theta); free(m); free(v); free(g); return -1; }

    if (h->fp32_param) memcpy(g, grad, bytes);
    else for (int64_t i = 0; i < n; ++i) g[i] = bf16_to_f32(((const uint16_t *)grad)[i]);

    if (h->quantize_states) {
        oracle_dequantize(m_codes, m_scales, n, momentum_spec(h->companded), m);
        oracle_dequantize(v_codes, v_scales, n, variance_spec(h->companded), v);
    } else {
        memcpy(m, m_codes, bytes);
        memcpy(v, v_codes, bytes);
    }

    if (h->fp32_param) memcpy(theta, param, bytes);
    else if (h->master_bits) oracle_reconstruct((const uint16_t *)param, rho, n, h->master_bits, theta);
    else for (int64_t i = 0; i < n; ++i) theta[i] = bf16_to_f32(((const uint16_t *)param)[i]);

    oracle_adamw_update(theta, m, v, g, n, h);

    if (h->quantize_states) {
        oracle_quantize(m, n, momentum_spec(h->companded), m_codes, m_scales);
        oracle_quantize(v, n, variance_spec(h->companded), v_codes, v_scales);
    } else {
        memcpy(m_codes, m, bytes);
        memcpy(v_codes, v, bytes);
    }

    if (h->fp32_param) memcpy(param, theta, bytes);
    else if (h->master_bits) oracle_split(theta, n, h->master_bits, (uint16_t *)param, rho);
    else for (int64_t i = 0; i < n; ++i) ((uint16_t *)param)[i] = bf16_rne(theta[i]);

    free(theta); free(m); free(v); free(g);
    return 0;
}

/* ------------------------------------------------------------- FlashSGD */

/* FlashSGD appears on the pages only through its memory accounting
 * ([SIM bytes_per_param()] "flash_sgd": bf16 master + rho + grad + one
 * group-32 quantized state of 1 + 2/32 bytes).  R16: its update is read as
 * torch.optim.SGD with momentum (the optimizer the page's "sgd_ref" row
 * accounts for), one fp32 operation per step, in torch's order:
 *   d   <- g + wd theta                         (coupled weight decay, if wd)
 *   buf <- d                                    at step 1,
 *   buf <- momentum buf + (1 - dampening) d     afterwards
 *   d   <- d + momentum buf  (nesterov)  or  d <- buf
 *   theta <- theta - lr d
 * and the momentum buffer is stored with the momentum spec of the codec
 * (the linear spec when !companded), the master split as for FlashAdamW. */
void oracle_sgd_update(float *theta, float *buf, const float *g, int64_t n,
                       const oracle_sgd_hparams *h)
{
    const float lr = (float)h->lr, mu = (float)h->momentum;
    const float wd = (float)h->weight_decay, cd = (float)(1.0 - h->dampening);
    for (int64_t i = 0; i < n; ++i) {
        float d = g[i];
        if (h->weight_decay != 0.0) {
            float decay = wd * theta[i];
            d = d + decay;
        }
        float b;
        if (h->step == 1) {
            b = d;
        } else {
            float kept = mu * buf[i];
            float added = cd * d;
            b = kept + added;
        }
        float dir;
        if (h->nesterov) {
            float look = mu * b;
            dir = d + look;
        } else {
            dir = b;
        }
        float upd = lr * dir;
        theta[i] = theta[i] - upd;
        buf[i] = b;
    }
}

int oracle_sgd_step(uint16_t *param, const uint16_t *grad, void *rho,
                    void *m_codes, uint16_t *m_scales, int64_t n,
                    const oracle_sgd_hparams *h)
{
    if (n < 0 || h == NULL || h->step < 1) return -1;
    if (h->master_bits != 0 && h->master_bits != 24 && h->master_bits != 32) return -1;
    if (n == 0) return 0;
    size_t bytes = (size_t)n * sizeof(float);
    float *theta = (float *)malloc(bytes), *m = (float *)malloc(bytes), *g = (float *)malloc(bytes);
    if (!theta || !m || !g) { free(theta); free(m); free(g); return -1; }

    for (int64_t i = 0; i < n; ++i) g[i] = bf16_to_f32(grad[i]);
    if (h->quantize_states) oracle_dequantize(m_codes, m_scales, n, momentum_spec(h->companded), m);
    else memcpy(m, m_codes, bytes);
    if (h->master_bits) oracle_reconstruct(param, rho, n, h->master_bits, theta);
    else for (int64_t i = 0; i < n; ++i) theta[i] = bf16_to_f32(param[i]);

    oracle_sgd_update(theta, m, g, n, h);

    if (h->quantize_states) oracle_quantize(m, n, momentum_spec(h->companded), m_codes, m_scales);
    else memcpy(m_codes, m, bytes);
    if (h->master_bits) oracle_split(theta, n, h->master_bits, param, rho);
    else for (int64_t i = 0; i < n; ++i) param[i] = bf16_rne(theta[i]);

    free(theta); free(m); free(g);
    return 0;
}

/* The list form used to time the oracle: every tensor is cut into slices of
 * SLICE elements (a multiple of the group, so no group is split) and the
 * slices are shared among OpenMP threads.  Each slice runs
 * oracle_adamw_step() unchanged. */
#define SLICE (GROUP * 1024)

static int run_slice(const oracle_tensor *q, int64_t s0, const oracle_hparams *h)
{
    size_t rho_elem = (h->master_bits == 32) ? 2 : 1;
    size_t state_elem = h->quantize_states ? 1 : sizeof(float);
    size_t param_elem = h->fp32_param ? sizeof(float) : sizeof(uint16_t);
    int64_t len = q->numel - s0 < SLICE ? q->numel - s0 : SLICE;
    void *rho = q->rho ? (char *)q->rho + (size_t)s0 * rho_elem : NULL;
    uint16_t *ms = h->quantize_states ? q->m_scales + s0 / GROUP : NULL;
    uint16_t *vs = h->quantize_states ? q->v_scales + s0 / GROUP : NULL;
    return oracle_adamw_step((char *)q->param + (size_t)s0 * param_elem,
                             (const char *)q->grad + (size_t)s0 * param_elem, rho,
                             (char *)q->m_codes + (size_t)s0 * state_elem, ms,
                             (char *)q->v_codes + (size_t)s0 * state_elem, vs,
                             len, h);
}

int oracle_adamw_step_list(const oracle_tensor *t, int n_tensors,
                           const oracle_hparams *h, int threads)
{
    if (n_tensors < 0 || (n_tensors > 0 && t == NULL) || h == NULL) return -1;
    int64_t total = 0;
    for (int i = 0; i < n_tensors; ++i) {
        if (t[i].numel < 0) return -1;
        total += (t[i].numel + SLICE - 1) / SLICE;
    }
    int64_t *owner = (int64_t *)malloc(sizeof(int64_t) * (size_t)(total + 1));
    int64_t *first = (int64_t *)malloc(sizeof(int64_t) * (size_t)(total + 1));
    if (!owner || !first) { free(owner); free(first); return -1; }
    int64_t w = 0;
    for (int i = 0; i < n_tensors; ++i)
        for (int64_t s = 0; s < t[i].numel; s += SLICE) { owner[w] = i; first[w] = s; ++w; }

    int used = 1, bad = 0;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#pragma omp parallel reduction(|:bad)
    {
#pragma omp single
        used = omp_get_num_threads();
#pragma omp for schedule(dynamic, 1)
        for (int64_t k = 0; k < total; ++k)
            bad |= (run_slice(&t[owner[k]], first[k], h) != 0);
    }
#else
    (void)threads;
    for (int64_t k = 0; k < total; ++k)
        bad |= (run_slice(&t[owner[k]], first[k], h) != 0);
#endif
    free(owner); free(first);
    return bad ? -1 : used;
}
