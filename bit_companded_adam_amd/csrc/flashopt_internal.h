// Internal declarations shared by the kernels (flashopt_kernels.hip) and the
// C-ABI host layer (flashopt_api.cpp) of libflashopt.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flashopt {

// Work decomposition: 1024-element chunks, 16 elements per lane of a
// 64-lane wavefront, processed in units of consecutive elements (the step
// kernels give each wavefront one unit, see the kernels); quantization
// groups are 32 elements; a 256-thread workgroup runs four wavefronts.
constexpr int kLaneElems = 16;
constexpr int kWaveLanes = 64;
constexpr int kChunkElems = kLaneElems * kWaveLanes;   // 1024
constexpr int kBlockThreads = 256;
constexpr int kGroup = 32;

// State storage of the step: codes with fp16 group scales under the linear or
// the companded specs, or plain fp32 moments (the unquantized-states ablation).
enum : int { kStatesLinear = 0, kStatesCompanded = 1, kStatesFp32 = 2 };

// The step kernels' parameter formats, as their master-bits argument: 24 and
// 32 split a bf16 parameter with int8 / int16 rho, 0 updates a bf16
// parameter without a split, kParamF32 updates an fp32 parameter (with an
// fp32 gradient) in place, never split.
constexpr int kParamF32 = 1;

// Per-tensor descriptor of the multi-tensor step, staged in the workspace.
// With fp32 states m_codes / v_codes point to float arrays.
struct DevTensor {
    uint16_t *param;
    const uint16_t *grad;
    void *rho;
    int8_t *m_codes;
    uint16_t *m_scales;
    uint8_t *v_codes;
    uint16_t *v_scales;
    int64_t numel;
};
static_assert(sizeof(DevTensor) == 64, "descriptor layout");

// Byte offsets of a chunk's state in the blocked state layout (bytes = 0:
// the per-tensor streams): block c of a tensor starts at rho + c * bytes and
// holds rho at 0, the m codes at m, the v codes at v, the m scales at ms and
// the v scales at vs.
struct StateLayout {
    uint32_t bytes, m, v, ms, vs;
};

// Scalars of one step.  The fp32 ones are formed in double on the host and
// rounded once (a Python float meeting a float32 tensor); rbc1 and inv_bc2s
// serve the kernel's exact short routes for the bias-correction quotients
// (div_markstein with rbc1; sqrt_quot_x2p32 with inv_bc2s).
struct StepScalars {
    double inv_bc2s;    // 2^64 / bc2 in double: vhat 2^64 inside sqrt_quot_x2p32
    float cwd;          // 1 - lr * wd
    float b1;           // beta1
    float c1;           // 1 - beta1
    float b2;           // beta2
    float c2;           // 1 - beta2
    float bc1;          // 1 - beta1^t
    float bc2;          // 1 - beta2^t
    float lr;
    float eps;
    float lr2;          // lr 2^32 (exact): the numerator's scale on the short route
    float eps2;         // eps 2^32 (exact): the denominator's scale on the short route
    float rbc1;         // 1 / bc1 correctly rounded to fp32
    float kv;           // 255 sqrt(bc2) 2^-32: the variance codes' factor from sqrt(vhat) 2^32
    float m1_max;       // |m1| up to this keeps |lr mhat 2^32| <= 2^100 eps2 and |m1| <= 2^99 bc1
    uint32_t v1_bound;  // v1 bit patterns below this keep vhat below 2^63
    uint32_t num_key;   // (pattern << 1) - 1 of the smallest nonzero |lr mhat 2^32| allowed
    int fast;           // 1 when eps and lr keep the short routes exact (see adamw_scalars)
    int unit_bc;        // bit 0: bc1 is exactly 1, bit 1: bc2 is exactly 1 (later in training)
    StateLayout blk;    // the state layout
};
// The list step kernels (AdamW and FlashSGD) read their scalars from device
// memory: a block of kScalarsBytes at the start of the staged table (the
// workspace, the allocation-free scratch array or a caller's plan), written
// by the same host-to-device copy as the table or by a later one, so that a
// launch can be captured once and replayed with new scalars.
constexpr size_t kScalarsBytes = 128;
static_assert(sizeof(StepScalars) <= kScalarsBytes, "scalar block");
// fp32 scalars of one FlashSGD step (SGD with momentum), formed in double
// on the host and rounded once.
struct SgdScalars {
    float lr;
    float mu;       // momentum
    float cd;       // 1 - dampening
    float wd;       // coupled weight decay
    int has_wd;     // weight_decay != 0
    int first;      // step == 1: the buffer is set to the gradient
    int nesterov;
    StateLayout blk;    // the state layout (no v parts)
};
static_assert(sizeof(SgdScalars) <= kScalarsBytes, "scalar block");

// Allocation-free list step: its scalar block and chunk table (up to
// kScratchTensors descriptors, then their chunk starts) live in a device
// array of the library, kScratchBytes long.  scratch_address returns that
// array's address on the current device (looked up once per device).
constexpr int kScratchTensors = 1024;
constexpr size_t kScratchBytes =
    (kScalarsBytes + sizeof(DevTensor) * kScratchTensors + sizeof(int32_t) * (kScratchTensors + 1) + 255) &
    ~size_t(255);
hipError_t scratch_address(void **ptr);

hipError_t launch_quantize(const float *x, int64_t n, unsigned spec, void *codes,
                           uint16_t *scales, hipStream_t stream);
hipError_t launch_dequantize(const void *codes, const uint16_t *scales, int64_t n,
                             unsigned spec, float *out, hipStream_t stream);
hipError_t launch_split(const float *master, int64_t n, int master_bits,
                        uint16_t *param, void *rho, hipStream_t stream);
hipError_t launch_reconstruct(const uint16_t *param, const void *rho, int64_t n,
                              int master_bits, float *master, hipStream_t stream);
// scalars / tensors / chunk_start are device pointers into the staged
// table; chunk_start has n_tensors + 1 entries.  master_bits: 24 | 32 | 0
// (no split) | kParamF32 (AdamW only); states: one of kStates*.
hipError_t launch_adamw_step(const StepScalars *scalars, const DevTensor *tensors,
                             const int32_t *chunk_start, int n_tensors, int32_t total_chunks,
                             int master_bits, int states, hipStream_t stream);
hipError_t launch_sgd_step(const SgdScalars *scalars, const DevTensor *tensors,
                           const int32_t *chunk_start, int n_tensors, int32_t total_chunks,
                           int master_bits, int states, hipStream_t stream);
// One tensor, its descriptor passed in the kernel arguments (no workspace).
hipError_t launch_adamw_tensor(const DevTensor &d, const StepScalars &sc, int master_bits,
                               int states, hipStream_t stream);
hipError_t launch_sgd_tensor(const DevTensor &d, const SgdScalars &sc, int master_bits,
                             int states, hipStream_t stream);

}  // namespace flashopt
