/*
 * Oracle for the FlashAdamW optimizer step: a plain, slow, single-purpose CPU
 * implementation of what the step computes, written from the method pages.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this code; only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg load it.  It shares no source with the HIP
 * library (no headers, helpers, tables or constants).
 *
 * Pages cited (titles as published):
 *   [EQ]  "code/gpu/equivalence.py"        -- battery(), eq_quantization(), eq_ecc()
 *   [QZ]  "code/flashsim/quantization.py"  -- module docstring (Alg. 2/3), _grouped(),
 *                                             quantize(), dequantize(), nmse()
 *   [SIM] "code/flashsim/flash_adamw_sim.py" -- FlashAdamWSim.step() (Alg. 4),
 *                                             bytes_per_param()
 *
 * Arithmetic: IEEE binary32, one rounding per operation (round to nearest
 * even), no contraction, subnormals kept -- what torch's eager CPU float32
 * ops do.  Host scalars are formed in double and rounded once to float, as a
 * Python float meets a float32 tensor.  Build with -ffp-contract=off
 * -fno-fast-math.
 *
 * Parity status: every function below is pinned by tests that do not re-type
 * its formula (closed forms, worked examples derived by hand under
 * tests/golden/, invariants, exhaustive checks, library routines).  The AdamW
 * body's operation order is pinned bit for bit by six hand-derived elements
 * whose stored bf16 half and rho change under each plausible reordering.
 * The multi-step values of oracle_adamw_step() with quantized states or the
 * 24-bit master are pinned by composition of pinned parts; over many steps
 * they are pinned independently only for groups of equal elements (whose
 * codes stay +-127 / 255, so the stored moments follow fp16 roundings of
 * closed form, for AdamW and FlashSGD): parity unpinned for the general
 * composite trajectory itself.  With fp32 moments and the 32-bit master a
 * 300-step trajectory is pinned to torch.optim.AdamW within a rounding
 * bound, and the fp32-parameter step equals the lossless 32-bit master step
 * bit for bit.
 */
#ifndef FLASHOPT_ORACLE_H
#define FLASHOPT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Quantizer spec flags, the three switches of quantize()/dequantize() [QZ]. */
#define ORACLE_SIGNED   1u
#define ORACLE_SQRT     2u
#define ORACLE_SOFTSIGN 4u

/* fp32 -> IEEE binary16 bits, round to nearest even, subnormals kept,
 * |x| >= 65520 -> +-Inf, NaN -> quiet NaN 0x7E00|sign.  This is the
 * fp16 cast that forms the per-group scale [QZ quantize()]. */
uint16_t oracle_f16_from_f32(float x);
/* The same conversion over an array. */
void oracle_f16_array(const float *x, int64_t n, uint16_t *out);
/* Exact widening of binary16 bits to fp32. */
float oracle_f32_from_f16(uint16_t h);

/* Weight split (Alg. 1; not printed on the pages, reading stated in the .c):
 * master fp32 -> (bf16 theta', rho).  master_bits 24 -> rho is int8,
 * 32 -> rho is int16.  Returns 0, or -1 for a bad master_bits. */
int oracle_split(const float *x, int64_t n, int master_bits,
                 uint16_t *theta_bf16, void *rho);
/* Inverse split: (theta', rho) -> fp32 master. */
int oracle_reconstruct(const uint16_t *theta_bf16, const void *rho, int64_t n,
                       int master_bits, float *x);

/* Group-32 absmax quantization with optional companding [QZ quantize()].
 * codes: n bytes (int8 when SIGNED, else uint8); scales: ceil(n/32) fp16
 * bits.  Returns 0. */
int oracle_quantize(const float *x, int64_t n, unsigned spec,
                    void *codes, uint16_t *scales);
/* Inverse [QZ dequantize()]. */
int oracle_dequantize(const void *codes, const uint16_t *scales, int64_t n,
                      unsigned spec, float *out);

/* Normalised MSE in double [QZ nmse()]. */
double oracle_nmse(const float *orig, const float *recon, int64_t n);

/* Hyper-parameters of one step, as the Python floats of [SIM]. */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    int64_t step;          /* t >= 1, the count after the increment */
    int master_bits;       /* 24 | 32 | 0 (0 = no split, plain bf16 param) */
    int companded;         /* 1: softsign m / sqrt v;  0: linear ablation */
    int quantize_states;   /* 1: int8/uint8 + fp16 scales;  0: fp32 m, v  */
    int fp32_param;        /* 1: fp32 parameter and gradient, never split
                              (needs master_bits 0);  0: bf16              */
} oracle_hparams;

/* The AdamW update alone (body of Alg. 4 [SIM step()]) on fp32 arrays, in
 * place: theta, m, v are read and overwritten; g is read. */
void oracle_adamw_update(float *theta, float *m, float *v, const float *g,
                         int64_t n, const oracle_hparams *h);

/* One FlashAdamW step on one parameter tensor [SIM step()], in place.
 * param/grad: bf16 bits [n], or float [n] with fp32_param.  rho: int8 [n]
 * (24) or int16 [n] (32), unused when master_bits == 0.  With quantize_states: m_codes int8 [n], m_scales
 * fp16 [ceil(n/32)], v_codes uint8 [n], v_scales fp16 [ceil(n/32)].  Without:
 * m_codes and v_codes point to float [n] states and the scale pointers are
 * unused.  Returns 0, or -1 on a bad argument. */
int oracle_adamw_step(void *param, const void *grad, void *rho,
                      void *m_codes, uint16_t *m_scales,
                      void *v_codes, uint16_t *v_scales,
                      int64_t n, const oracle_hparams *h);

/* FlashSGD hyper-parameters (R16 in flashopt_oracle.c: torch.optim.SGD with
 * momentum, the momentum buffer stored with the momentum spec). */
typedef struct {
    double lr, momentum, dampening, weight_decay;
    int64_t step;          /* t >= 1; step 1 sets the buffer to the gradient */
    int master_bits;       /* 24 | 32 | 0 */
    int companded;         /* 1: softsign momentum spec;  0: linear         */
    int quantize_states;   /* 1: int8 + fp16 scales;  0: fp32 buffer        */
    int nesterov;
} oracle_sgd_hparams;

/* The SGD-with-momentum update alone on fp32 arrays, in place. */
void oracle_sgd_update(float *theta, float *buf, const float *g, int64_t n,
                       const oracle_sgd_hparams *h);

/* One FlashSGD step on one tensor, in place (layouts as oracle_adamw_step,
 * with the momentum buffer in m_codes / m_scales).  Returns 0, or -1 on a
 * bad argument. */
int oracle_sgd_step(uint16_t *param, const uint16_t *grad, void *rho,
                    void *m_codes, uint16_t *m_scales, int64_t n,
                    const oracle_sgd_hparams *h);

/* The same step over a list of tensors, split into 32-aligned slices that
 * run on `threads` OpenMP threads (<= 0: the runtime default).  Used to time
 * the oracle; the arithmetic is oracle_adamw_step()'s.  Returns the thread
 * count used, or -1 on a bad argument. */
typedef struct {
    void *param; const void *grad; void *rho;
    void *m_codes; uint16_t *m_scales; void *v_codes; uint16_t *v_scales;
    int64_t numel;
} oracle_tensor;
int oracle_adamw_step_list(const oracle_tensor *t, int n_tensors,
                           const oracle_hparams *h, int threads);

#ifdef __cplusplus
}
#endif
#endif
