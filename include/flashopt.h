/*
 * flashopt.h -- C ABI of libflashopt.so, the MI355X (gfx950) FlashAdamW and
 * FlashSGD steps.
 *
 * The method is described on the pages
 *   "code/flashsim/quantization.py"    (group-32 companded int8/uint8 state codec,
 *                                      Alg. 2 momentum / Alg. 3 variance),
 *   "code/flashsim/flash_adamw_sim.py" (FlashAdamWSim.step: Alg. 4, the step),
 *   "code/gpu/equivalence.py"          (the bf16 parameter and its correction
 *                                      bits rho, eq_ecc()).
 *
 * Conventions for every entry point:
 *   - Buffer pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates or frees device memory and keeps no state between calls
 *     except a small cache of pinned host staging buffers (see
 *     flashopt_adamw_step) and the allocation-free step's static table (see
 *     flashopt_adamw_step_noalloc).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  Results are visible after the stream is synchronized.
 *     The stream and every buffer belong to the calling thread's current HIP
 *     device (hipSetDevice); calls from several threads are safe.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     status other than FLASHOPT_OK means nothing was launched.  Faults inside
 *     a kernel surface at the caller's next synchronization.
 *   - n == 0 is a no-op that returns FLASHOPT_OK (pointers may then be NULL).
 *   - Groups of 32 elements start at element 0 of every array; a ragged last
 *     group behaves as if padded with zeros (page "code/flashsim/quantization.py",
 *     _grouped()).  Scale arrays hold ceil(n / 32) entries.
 *   - fp16 and bf16 values are passed as their uint16_t bit patterns.
 *   - Non-finite inputs are outside the contract; the results stay defined
 *     (NaN codes are 0) but are not part of the parity guarantee.
 *   - Input and output buffers must not overlap, except where a call says it
 *     updates a buffer in place.
 *   - Alignment: every element stream (fp32, bf16, codes, rho) must start on a
 *     16-byte boundary, scale arrays on a 2-byte boundary; otherwise
 *     FLASHOPT_EALIGN.  Allocations from hipMalloc / torch satisfy this.
 *   - A step call launches its step kernel once.  A list (or tensor) of more
 *     than 2^25 - 2 chunks of 1024 elements (2^24 - 1 with fp32 states or
 *     fp32 parameters) does not fit one dispatch's 32-bit count of
 *     work-items and is stepped by one launch per such range of chunks, in
 *     order on the same stream.  Should a later launch of such a split fail,
 *     the earlier ones have already been enqueued.
 */
#ifndef FLASHOPT_H
#define FLASHOPT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLASHOPT_ABI_VERSION 8

typedef enum {
    FLASHOPT_OK = 0,
    FLASHOPT_EINVAL = 1,      /* an argument is out of its documented range      */
    FLASHOPT_EALIGN = 2,      /* a buffer violates the alignment rule above      */
    FLASHOPT_EWORKSPACE = 3,  /* the workspace or plan buffer is NULL or too small,
                                 or a list exceeds a fixed table (noalloc)   */
    FLASHOPT_EHIP = 4         /* the HIP runtime reported an error on enqueue    */
} flashopt_status;

/* Quantizer spec bits: the three switches of quantize()/dequantize() on page
 * "code/flashsim/quantization.py". */
enum {
    FLASHOPT_Q_SIGNED = 1u,   /* int8 codes in [-127, 127] from max |x|; else uint8 [0, 255] from max x */
    FLASHOPT_Q_SQRT = 2u,     /* quantize sqrt(x), dequantize to the square              */
    FLASHOPT_Q_SOFTSIGN = 4u  /* compand y -> 2y / (1 + |y|), inverse y -> y / (2 - |y|) */
};
/* The named specs of that page: Alg. 2 momentum, Alg. 3 variance, and the
 * linear ablation of both (no companding). */
#define FLASHOPT_SPEC_MOMENTUM        (FLASHOPT_Q_SIGNED | FLASHOPT_Q_SOFTSIGN)
#define FLASHOPT_SPEC_VARIANCE        (FLASHOPT_Q_SQRT)
#define FLASHOPT_SPEC_MOMENTUM_LINEAR (FLASHOPT_Q_SIGNED)
#define FLASHOPT_SPEC_VARIANCE_LINEAR (0u)

/* Group-32 absmax quantization with optional companding (page
 * "code/flashsim/quantization.py", quantize(); Alg. 2/3 forward).  Per group:
 * a = sqrt(x) if SQRT; s = fp16(max |a|) (SIGNED) or fp16(max a); d = 1 if s is
 * zero else s; y = a / d; y = 2y / (1 + |y|) if SOFTSIGN; code = round half to
 * even of y*127 clamped to [-127, 127] (SIGNED) or of y*255 clamped to [0, 255].
 *   x      [n] fp32, read
 *   spec   any OR of FLASHOPT_Q_* bits (bits above 7 -> EINVAL)
 *   codes  [n] int8 (SIGNED) or uint8, written
 *   scales [ceil(n/32)] fp16 bits, written
 * Errors: EINVAL (n < 0, NULL pointer with n > 0, bad spec), EALIGN, EHIP. */
flashopt_status flashopt_quantize(const float *x, int64_t n, unsigned spec,
                                  void *codes, uint16_t *scales, void *stream);

/* Inverse (page "code/flashsim/quantization.py", dequantize()): y = q/127 or
 * q/255; y = y / (2 - |y|) if SOFTSIGN; out = y * s; out = out * out if SQRT.
 *   codes [n] int8|uint8 and scales [ceil(n/32)] fp16 bits, read
 *   out   [n] fp32, written
 * Errors: as flashopt_quantize. */
flashopt_status flashopt_dequantize(const void *codes, const uint16_t *scales,
                                    int64_t n, unsigned spec, float *out,
                                    void *stream);

/* Weight split, Alg. 1 (called but not printed on page
 * "code/flashsim/flash_adamw_sim.py"; the bf16 parameter and correction bits
 * rho of page "code/gpu/equivalence.py", eq_ecc()).  This library's reading:
 *   theta' = master rounded to the nearest bf16, ties away from zero;
 *   D      = bit pattern of master minus (bit pattern of theta') << 16,
 *            D in [-32768, 32767];
 *   rho    = D (master_bits 32, int16: lossless for every non-NaN input), or
 *            D/256 rounded half to even and clamped to [-128, 127]
 *            (master_bits 24, int8: within 128 fp32 ulps, 255 when D >= 32640).
 *   NaN: theta' keeps the upper half with the quiet bit set, rho = 0.
 *   master [n] fp32, read;  param_bf16 [n] written;  rho [n] int8|int16 written
 * Errors: EINVAL (also master_bits not 24 or 32), EALIGN, EHIP. */
flashopt_status flashopt_split(const float *master, int64_t n, int master_bits,
                               uint16_t *param_bf16, void *rho, void *stream);

/* Inverse split: bit pattern of master = (theta' << 16) + rho * 2^(16 - w),
 * w = 8 (24-bit master) or 16 (32-bit), in wrapping 32-bit integer arithmetic.
 *   param_bf16 [n], rho [n] read;  master [n] fp32 written
 * Errors: as flashopt_split. */
flashopt_status flashopt_reconstruct(const uint16_t *param_bf16, const void *rho,
                                     int64_t n, int master_bits, float *master,
                                     void *stream);

/* One parameter tensor of a FlashAdamW step (page
 * "code/flashsim/flash_adamw_sim.py", FlashAdamWSim.step: per-parameter state
 * m = (codes, scales), v = (codes, scales), rho).  All device pointers.
 * param, rho, m_*, v_* are read and updated in place; grad is read only.
 * Fresh state is all zero (codes, scales, fp32 moments and rho), which
 * reproduces the page's state init for a bf16 parameter.
 * With args.fp32_states = 1 (the page's quantize_states=False ablation),
 * m_codes and v_codes point to float [numel] moments and the scale pointers
 * are unused (may be NULL).  With args.master_bits = 0 (the page's
 * master_weight_bits=None) rho is unused (may be NULL).
 *
 * State layouts (args.state_layout).  FLASHOPT_STATE_STREAMS: rho, m_codes,
 * m_scales, v_codes and v_scales are five arrays as above (the page's
 * per-parameter tensors).  FLASHOPT_STATE_BLOCKED: the same values, stored
 * chunk by chunk in one buffer that `rho` points to (16-byte aligned; the
 * other four state pointers must be NULL): ceil(numel / 1024) blocks of
 * equal size in chunk order, each padded to a multiple of 128 bytes (one
 * cache line never holds two chunks' state), block c holding, for elements
 * 1024 c .. 1024 c + 1023,
 *   rho      1024 bytes (24-bit master) | 2048 (32-bit) | none (no split)
 *   m codes  1024 bytes
 *   v codes  1024 bytes                      (AdamW only)
 *   m scales 32 fp16 (64 bytes)
 *   v scales 32 fp16 (64 bytes)              (AdamW only)
 * (flashopt_blocked_state_bytes gives the buffer size).  Bytes past numel in
 * the last block are neither read nor written.  The step then reads and
 * writes three regions per chunk (parameter, gradient, state block) instead
 * of seven arrays; the arithmetic and every stored value are the same.
 * Quantized states only (not with fp32_states). */
enum {
    FLASHOPT_STATE_STREAMS = 0,
    FLASHOPT_STATE_BLOCKED = 1
};
typedef struct {
    uint16_t *param;          /* [numel] bf16 theta'                          */
    const uint16_t *grad;     /* [numel] bf16 gradient                        */
    void *rho;                /* [numel] int8 (24-bit) | int16 (32-bit)       */
    int8_t *m_codes;          /* [numel] momentum codes (fp32 states: float)  */
    uint16_t *m_scales;       /* [ceil(numel/32)] fp16 momentum scales        */
    uint8_t *v_codes;         /* [numel] variance codes (fp32 states: float)  */
    uint16_t *v_scales;       /* [ceil(numel/32)] fp16 variance scales        */
    int64_t numel;            /* >= 0                                         */
} flashopt_tensor;

/* Step hyper-parameters, as the Python floats of FlashAdamWSim. */
typedef struct {
    double lr;                /* >= 0                                         */
    double beta1, beta2;      /* in [0, 1)                                    */
    double eps;               /* >= 0                                         */
    double weight_decay;      /* finite; decoupled: theta *= 1 - lr * wd      */
    int64_t step;             /* t >= 1, the step count after this step's increment */
    int master_bits;          /* 24 (int8 rho) | 32 (int16 rho) | 0: no split,
                                 the bf16 parameter itself is the master and
                                 the update is cast back to bf16 rounding to
                                 nearest even (master_weight_bits=None)      */
    int companded;            /* 1: softsign m, sqrt v (Alg. 2/3); 0: linear ablation */
    int fp32_states;          /* 0: quantized m, v (codes + fp16 scales);
                                 1: fp32 m, v (quantize_states=False)         */
    int param_fp32;           /* 0: bf16 parameters and gradients;
                                 1: fp32 parameters and fp32 gradients (param
                                 and grad point to float [numel]), never split
                                 (the page's use_split is false for an fp32
                                 parameter): theta is the parameter and the
                                 update is stored unchanged; needs
                                 master_bits 0 (rho unused)                   */
    int state_layout;         /* FLASHOPT_STATE_STREAMS | FLASHOPT_STATE_BLOCKED */
} flashopt_adamw_args;

/* Bytes of a FLASHOPT_STATE_BLOCKED state buffer for a tensor of numel
 * elements: ceil(numel / 1024) blocks of (rho bytes for master_bits 24 | 32
 * | 0: 1024 | 2048 | 0) + 1024 + 64 bytes, plus 1024 + 64 with_variance
 * (AdamW: 1; FlashSGD: 0), rounded up to a multiple of 128.  Returns 0 for
 * numel <= 0 or another master_bits. */
size_t flashopt_blocked_state_bytes(int64_t numel, int master_bits, int with_variance);

/* Device workspace bytes that flashopt_adamw_step needs for this list (the
 * step's scalar block, then the per-tensor descriptor and chunk table).
 * Returns 0 for n_tensors <= 0. */
size_t flashopt_adamw_workspace_bytes(const flashopt_tensor *tensors, int n_tensors);

/* One fused FlashAdamW step over a list of tensors, one kernel launch (see
 * the conventions for lists too long for one dispatch) (page
 * "code/flashsim/flash_adamw_sim.py", FlashAdamWSim.step, Alg. 4).  Per
 * element, in one pass over memory:
 *   m0 = dequantize(m), v0 = dequantize(v)      (momentum / variance spec, or
 *                                                 the linear specs if !companded;
 *                                                 fp32 states are read as is)
 *   theta = reconstruct(param, rho)             (the bf16 param if master_bits 0)
 *   theta *= 1 - lr*wd;  m1 = b1 m0 + (1-b1) g;  v1 = b2 v0 + ((1-b2) g) g
 *   mhat = m1 / (1 - b1^t);  vhat = v1 / (1 - b2^t)
 *   theta -= (lr mhat) / (sqrt(vhat) + eps)     (the page's order, "Standard
 *                                                 AdamW update")
 *   (m, v) = quantize(m1), quantize(v1);  (param, rho) = split(theta)
 *   (fp32 states: m, v = m1, v1;  master_bits 0: param = bf16 RNE of theta;
 *    param_fp32: theta = param, param = theta)
 * Scalars are formed in double on the host and rounded once to fp32; every
 * fp32 operation is rounded once, in the order written (no contraction).
 *   tensors   HOST array of n_tensors descriptors (read during the call only)
 *   workspace DEVICE buffer of at least flashopt_adamw_workspace_bytes();
 *             overwritten; it must not be reused by another call until this
 *             step has run on `stream`
 * The scalars and the descriptor table are staged through a pinned host
 * buffer that the library allocates once and reuses (hipHostMalloc).  That
 * staging is an ordinary asynchronous host-to-device copy from reused
 * memory, so a call captured into a HIP graph would replay whatever the
 * buffer holds at replay time: do not capture this call; the plan calls
 * below are its capture-safe form.  flashopt_adamw_step_tensor launches one
 * kernel with its arguments by value and stages nothing.
 * Errors: EINVAL (n_tensors < 0, NULL tensors/args, numel < 0, NULL pointer
 * that the variant uses in a non-empty tensor, master_bits, companded,
 * fp32_states, param_fp32, state_layout not 0 or 1, param_fp32 with
 * master_bits != 0, a blocked layout with fp32_states or with a non-NULL
 * m_codes, m_scales, v_codes or v_scales,
 * step < 1, lr < 0, beta outside
 * [0, 1), eps < 0, non-finite weight_decay, more than 2^31 - 1 chunks of
 * 1024 elements in total), EALIGN, EWORKSPACE, EHIP. */
flashopt_status flashopt_adamw_step(const flashopt_tensor *tensors, int n_tensors,
                                    const flashopt_adamw_args *args,
                                    void *workspace, size_t workspace_bytes,
                                    void *stream);

/* flashopt_adamw_step for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, results and validation as flashopt_adamw_step, without a
 * workspace: the scalars and the chunk table go to a device array inside
 * the library (68 KiB per GPU, held until the process ends) through one pageable
 * hipMemcpyAsync from a static host buffer, and the call allocates nothing
 * (no hipMalloc, hipHostMalloc, hipFree or event creation; the first call on
 * a device looks the array's address up once).
 * Limit: at most 1024 tensors per call (more -> FLASHOPT_EWORKSPACE, nothing
 * launched).  Every call on a GPU shares that GPU's array, which keeps the
 * last call's table: calls on one stream are ordered, but calls that overlap
 * on one GPU (different streams, or a second process thread's stream before
 * the first call's kernel ran) race on it.  The host buffer is guarded by a
 * mutex; the copy reads host memory at the call, so the call is not
 * capturable into a graph as is.
 * Errors: as flashopt_adamw_step (EWORKSPACE only for n_tensors > 1024). */
flashopt_status flashopt_adamw_step_noalloc(const flashopt_tensor *tensors, int n_tensors,
                                            const flashopt_adamw_args *args, void *stream);

/* A capture-safe form of flashopt_adamw_step, for a training step captured
 * into a HIP graph: the scalar block and the descriptor and chunk tables
 * live in a caller-owned DEVICE buffer (the plan), and the launch reads them
 * there.  Results are those of flashopt_adamw_step with the same tensors and
 * arguments.
 *
 * flashopt_adamw_plan_bytes(n): bytes of a plan for n tensors (the same as
 *   flashopt_adamw_workspace_bytes; 0 for n <= 0).
 * flashopt_adamw_plan(tensors, n, args, plan, plan_bytes, info, stream):
 *   validates the list and args as flashopt_adamw_step does, enqueues one
 *   host-to-device copy on `stream` that writes the scalars of args->step
 *   and the tables into `plan` (16-byte aligned), and fills *info (a host
 *   struct: list size and the variant fields of args).  The tensors' buffers
 *   must stay where they are for as long as the plan is launched.
 * flashopt_adamw_plan_set_step(info, args, plan, stream): enqueues one
 *   128-byte host-to-device copy of the scalars of args (any step and
 *   hyper-parameters; master_bits, companded, fp32_states, param_fp32 and
 *   state_layout must equal the plan's, else EINVAL).
 * flashopt_adamw_plan_launch(info, plan, stream): enqueues the step kernel
 *   only.  It copies nothing, allocates nothing and does not synchronize, so
 *   it can be captured into a graph; a launch or graph replay steps with the
 *   scalars that the last plan / plan_set_step copy wrote before it runs.
 * The two staging calls copy from library-owned pinned buffers at the call
 * and must not be captured: between replays, call plan_set_step with the
 * next step count on the replay stream (or one ordered before it), then
 * replay.  `info` must be the one flashopt_adamw_plan filled for `plan`.
 * Errors: as flashopt_adamw_step (EWORKSPACE: plan NULL or smaller than
 * flashopt_adamw_plan_bytes; EINVAL also for a NULL info or a variant
 * mismatch). */
size_t flashopt_adamw_plan_bytes(int n_tensors);
typedef struct {
    int32_t n_tensors;        /* tensors in the plan's table                  */
    int32_t total_chunks;     /* their 1024-element chunks                    */
    int32_t master_bits;      /* the variant fields of the planning args      */
    int32_t companded;
    int32_t fp32_states;
    int32_t param_fp32;
    int32_t state_layout;
} flashopt_adamw_plan_info;
flashopt_status flashopt_adamw_plan(const flashopt_tensor *tensors, int n_tensors,
                                    const flashopt_adamw_args *args, void *plan,
                                    size_t plan_bytes, flashopt_adamw_plan_info *info,
                                    void *stream);
flashopt_status flashopt_adamw_plan_set_step(const flashopt_adamw_plan_info *info,
                                             const flashopt_adamw_args *args, void *plan,
                                             void *stream);
flashopt_status flashopt_adamw_plan_launch(const flashopt_adamw_plan_info *info,
                                           const void *plan, void *stream);

/* FlashSGD hyper-parameters.  FlashSGD appears on page
 * "code/flashsim/flash_adamw_sim.py" only in bytes_per_param ("flash_sgd":
 * bf16 master + rho + grad + one group-32 state of 1 + 2/32 bytes); this
 * library reads its update as torch.optim.SGD with momentum, in torch's
 * order, one fp32 rounding per operation:
 *   d   = g + weight_decay * theta                 (coupled; skipped if 0)
 *   buf = d at step 1, else momentum * buf + (1 - dampening) * d
 *   dir = d + momentum * buf if nesterov, else buf
 *   theta = theta - lr * dir
 * with the buffer stored under the momentum spec (softsign int8, or the
 * linear spec if !companded) or as fp32, and the master split as for
 * flashopt_adamw_step. */
typedef struct {
    double lr;                /* >= 0                                         */
    double momentum;          /* > 0 (plain SGD keeps no state to compress)   */
    double dampening;         /* finite; must be 0 with nesterov              */
    double weight_decay;      /* finite                                       */
    int64_t step;             /* t >= 1; step 1 sets the buffer to d          */
    int master_bits;          /* 24 | 32 | 0 (no split), as flashopt_adamw_args */
    int companded;            /* 1: softsign momentum spec; 0: linear         */
    int fp32_states;          /* 0: codes + fp16 scales; 1: fp32 buffer       */
    int nesterov;             /* 0 | 1                                        */
    int state_layout;         /* FLASHOPT_STATE_STREAMS | FLASHOPT_STATE_BLOCKED
                                 (the blocked buffer without the v parts)     */
} flashopt_sgd_args;

/* Device workspace bytes that flashopt_sgd_step needs for this list. */
size_t flashopt_sgd_workspace_bytes(const flashopt_tensor *tensors, int n_tensors);

/* One fused FlashSGD step over a list of tensors, one kernel launch (see the
 * conventions for lists too long for one dispatch).  The
 * momentum buffer lives in each descriptor's m_codes / m_scales (or in the
 * blocked buffer at rho); v_codes and v_scales are unused (may be NULL;
 * NULL with the blocked layout).  Ownership, staging, workspace and
 * alignment rules as flashopt_adamw_step.
 * Errors: EINVAL (as flashopt_adamw_step for the list; momentum <= 0,
 * non-finite dampening or weight_decay, nesterov with dampening != 0, bad
 * nesterov / companded / fp32_states / master_bits / state_layout, step < 1,
 * lr < 0),
 * EALIGN, EWORKSPACE, EHIP. */
flashopt_status flashopt_sgd_step(const flashopt_tensor *tensors, int n_tensors,
                                  const flashopt_sgd_args *args,
                                  void *workspace, size_t workspace_bytes,
                                  void *stream);

/* The capture-safe form of flashopt_sgd_step, with the contract of the
 * flashopt_adamw_plan calls above: flashopt_sgd_plan stages the scalars of
 * args and the tables into `plan` (flashopt_sgd_plan_bytes(n) bytes) and
 * fills *info; flashopt_sgd_plan_set_step rewrites the scalars (any step and
 * hyper-parameters; master_bits, companded, fp32_states and state_layout
 * must equal the plan's); flashopt_sgd_plan_launch enqueues the kernel only
 * and can be captured into a graph.
 * Errors: as flashopt_sgd_step (EWORKSPACE for a NULL or short plan; EINVAL
 * also for a NULL info or a variant mismatch). */
size_t flashopt_sgd_plan_bytes(int n_tensors);
typedef struct {
    int32_t n_tensors;        /* tensors in the plan's table                  */
    int32_t total_chunks;     /* their 1024-element chunks                    */
    int32_t master_bits;      /* the variant fields of the planning args      */
    int32_t companded;
    int32_t fp32_states;
    int32_t state_layout;
} flashopt_sgd_plan_info;
flashopt_status flashopt_sgd_plan(const flashopt_tensor *tensors, int n_tensors,
                                  const flashopt_sgd_args *args, void *plan, size_t plan_bytes,
                                  flashopt_sgd_plan_info *info, void *stream);
flashopt_status flashopt_sgd_plan_set_step(const flashopt_sgd_plan_info *info,
                                           const flashopt_sgd_args *args, void *plan,
                                           void *stream);
flashopt_status flashopt_sgd_plan_launch(const flashopt_sgd_plan_info *info, const void *plan,
                                         void *stream);

/* One tensor's FlashAdamW / FlashSGD step without a workspace: the
 * descriptor travels in the kernel arguments, so the call stages nothing and
 * enqueues one kernel launch (see the conventions for a tensor too long for
 * one dispatch).  Meant for launching each tensor's step as
 * soon as its gradient is complete (gradient release: a post-accumulate-grad
 * hook steps the parameter and frees its gradient, so a full set of
 * gradients is never held; page "code/flashsim/flash_adamw_sim.py",
 * bytes_per_param(gradient_release=True)).  Results are identical to the
 * list forms for that tensor.
 *   tensor  HOST pointer to one descriptor (read during the call only)
 * Errors: as the list forms (EINVAL, EALIGN, EHIP; no EWORKSPACE). */
flashopt_status flashopt_adamw_step_tensor(const flashopt_tensor *tensor,
                                           const flashopt_adamw_args *args, void *stream);
flashopt_status flashopt_sgd_step_tensor(const flashopt_tensor *tensor,
                                         const flashopt_sgd_args *args, void *stream);

/* Static string naming a status code. */
const char *flashopt_status_str(flashopt_status status);

/* FLASHOPT_ABI_VERSION of the loaded library. */
int flashopt_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FLASHOPT_H */
