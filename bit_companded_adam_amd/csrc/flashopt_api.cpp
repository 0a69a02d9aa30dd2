// C-ABI host layer of libflashopt.so: argument validation, the multi-tensor
// chunk table, step scalars, and kernel launches on the caller's stream.
// Every entry point validates everything before it enqueues anything, and no
// C++ exception crosses the ABI.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>

#include "flashopt.h"
#include "flashopt_internal.h"

namespace {

using flashopt::DevTensor;
using flashopt::SgdScalars;
using flashopt::StepScalars;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

flashopt_status hip_status(hipError_t e) { return e == hipSuccess ? FLASHOPT_OK : FLASHOPT_EHIP; }

flashopt_status check_codec(const void *elems, int64_t n, unsigned spec, const void *codes,
                            const uint16_t *scales)
{
    if (n < 0 || spec > 7u) return FLASHOPT_EINVAL;
    if (n == 0) return FLASHOPT_OK;
    if (!elems || !codes || !scales) return FLASHOPT_EINVAL;
    if (!aligned(elems, 16) || !aligned(codes, 16) || !aligned(scales, 2)) return FLASHOPT_EALIGN;
    return FLASHOPT_OK;
}

flashopt_status check_split(const void *master, int64_t n, int master_bits, const void *param,
                            const void *rho)
{
    if (n < 0 || (master_bits != 24 && master_bits != 32)) return FLASHOPT_EINVAL;
    if (n == 0) return FLASHOPT_OK;
    if (!master || !param || !rho) return FLASHOPT_EINVAL;
    if (!aligned(master, 16) || !aligned(param, 16) || !aligned(rho, 16)) return FLASHOPT_EALIGN;
    return FLASHOPT_OK;
}

// Table layout: [n DevTensor][n + 1 int32 chunk starts], 16-byte rounded.
size_t table_bytes(int n)
{
    if (n <= 0) return 0;
    size_t b = sizeof(DevTensor) * static_cast<size_t>(n) + sizeof(int32_t) * (static_cast<size_t>(n) + 1);
    return (b + 15) & ~static_cast<size_t>(15);
}

// Staged bytes of a list step: a header (the step's scalar block), then the
// table.
size_t staged_bytes(int n, size_t header_bytes)
{
    return n <= 0 ? 0 : header_bytes + table_bytes(n);
}

constexpr size_t kHeader = flashopt::kScalarsBytes;

// The scalar block of a list step: its StepScalars or SgdScalars, zero
// padded.
template <typename Sc>
void fill_scalars(const Sc &sc, void *dst)
{
    static_assert(sizeof(Sc) <= kHeader, "scalar block");
    std::memset(dst, 0, kHeader);
    std::memcpy(dst, &sc, sizeof(sc));
}

// Pinned host staging for the chunk table: a small ring per device, so the
// host can run a few steps ahead of the GPU.  A slot is reused only after
// the copy that last read it has completed.
constexpr int kRingSlots = 4;
constexpr int kMaxDevices = 64;

struct Slot {
    void *host = nullptr;
    size_t cap = 0;
    hipEvent_t done = nullptr;
    bool pending = false;
};

struct Ring {
    Slot slot[kRingSlots];
    int next = 0;
};

std::mutex g_ring_mutex;
Ring g_rings[kMaxDevices];

// Validation of one tensor of a step.  split: rho is used; quant: scales are
// used; v: the variance streams are used; blocked: the state is one
// chunk-blocked buffer at rho, and the other state pointers are NULL.
flashopt_status check_tensor(const flashopt_tensor &t, bool split, bool quant, bool v, bool blocked)
{
    if (t.numel < 0) return FLASHOPT_EINVAL;
    if (t.numel == 0) return FLASHOPT_OK;
    if (!t.param || !t.grad) return FLASHOPT_EINVAL;
    if (blocked) {
        if (!t.rho || t.m_codes || t.m_scales || t.v_codes || t.v_scales) return FLASHOPT_EINVAL;
        if (!aligned(t.param, 16) || !aligned(t.grad, 16) || !aligned(t.rho, 16)) return FLASHOPT_EALIGN;
    } else {
        if (!t.m_codes) return FLASHOPT_EINVAL;
        if (v && !t.v_codes) return FLASHOPT_EINVAL;
        if (split && !t.rho) return FLASHOPT_EINVAL;
        if (quant && (!t.m_scales || (v && !t.v_scales))) return FLASHOPT_EINVAL;
        if (!aligned(t.param, 16) || !aligned(t.grad, 16) || !aligned(t.m_codes, 16))
            return FLASHOPT_EALIGN;
        if (v && !aligned(t.v_codes, 16)) return FLASHOPT_EALIGN;
        if (split && !aligned(t.rho, 16)) return FLASHOPT_EALIGN;
        if (quant && (!aligned(t.m_scales, 2) || (v && !aligned(t.v_scales, 2)))) return FLASHOPT_EALIGN;
    }
    if ((t.numel + flashopt::kChunkElems - 1) / flashopt::kChunkElems > INT32_MAX) return FLASHOPT_EINVAL;
    return FLASHOPT_OK;
}

// Rho bytes of one 1024-element chunk: int8 or int16 correction bits, none
// without a split (master_bits 0).
uint32_t chunk_rho_bytes(int master_bits)
{
    return master_bits == 24 ? 1024u : (master_bits == 32 ? 2048u : 0u);
}

// The byte offsets of the blocked state layout (all zero for the streams):
// per chunk rho, m codes, v codes (with_v), m scales, v scales (with_v), the
// block padded to whole 128-byte cache lines, so that no line holds the
// state of two chunks (two wavefronts).
flashopt::StateLayout state_layout(int layout, int master_bits, bool with_v)
{
    flashopt::StateLayout L{0u, 0u, 0u, 0u, 0u};
    if (layout != FLASHOPT_STATE_BLOCKED) return L;
    const uint32_t r = chunk_rho_bytes(master_bits);
    const uint32_t codes = flashopt::kChunkElems;                          // one byte each
    const uint32_t scales = flashopt::kChunkElems / flashopt::kGroup * 2;  // fp16 each
    L.m = r;
    if (with_v) {
        L.v = r + codes;
        L.ms = r + 2 * codes;
        L.vs = r + 2 * codes + scales;
        L.bytes = r + 2 * codes + 2 * scales;
    } else {
        L.ms = r + codes;
        L.bytes = r + codes + scales;
    }
    L.bytes = (L.bytes + 127u) & ~127u;
    return L;
}

DevTensor device_descriptor(const flashopt_tensor &s)
{
    DevTensor d;
    d.param = s.param;
    d.grad = s.grad;
    d.rho = s.rho;
    d.m_codes = s.m_codes;
    d.m_scales = s.m_scales;
    d.v_codes = s.v_codes;
    d.v_scales = s.v_scales;
    d.numel = s.numel;
    return d;
}

int states_of(int fp32_states, int companded)
{
    return fp32_states ? flashopt::kStatesFp32
                       : (companded ? flashopt::kStatesCompanded : flashopt::kStatesLinear);
}

// The step kernels' parameter format: the master width, or kParamF32.
int kernel_format(const flashopt_adamw_args &a)
{
    return a.param_fp32 ? flashopt::kParamF32 : a.master_bits;
}

// AdamW hyper-parameters checked, then the step's fp32 scalars formed in
// double and rounded once.
flashopt_status adamw_scalars(const flashopt_adamw_args *a, StepScalars &sc)
{
    if (!a) return FLASHOPT_EINVAL;
    if (a->master_bits != 24 && a->master_bits != 32 && a->master_bits != 0) return FLASHOPT_EINVAL;
    if (a->companded != 0 && a->companded != 1) return FLASHOPT_EINVAL;
    if (a->fp32_states != 0 && a->fp32_states != 1) return FLASHOPT_EINVAL;
    if (a->param_fp32 != 0 && a->param_fp32 != 1) return FLASHOPT_EINVAL;
    if (a->param_fp32 && a->master_bits != 0) return FLASHOPT_EINVAL;
    if (a->state_layout != FLASHOPT_STATE_STREAMS && a->state_layout != FLASHOPT_STATE_BLOCKED)
        return FLASHOPT_EINVAL;
    if (a->state_layout == FLASHOPT_STATE_BLOCKED && a->fp32_states) return FLASHOPT_EINVAL;
    if (a->step < 1) return FLASHOPT_EINVAL;
    if (!(a->lr >= 0.0) || !std::isfinite(a->lr)) return FLASHOPT_EINVAL;
    if (!(a->beta1 >= 0.0 && a->beta1 < 1.0) || !(a->beta2 >= 0.0 && a->beta2 < 1.0)) return FLASHOPT_EINVAL;
    if (!(a->eps >= 0.0) || !std::isfinite(a->eps)) return FLASHOPT_EINVAL;
    if (!std::isfinite(a->weight_decay)) return FLASHOPT_EINVAL;
    const double t = static_cast<double>(a->step);
    sc.blk = state_layout(a->state_layout, a->master_bits, true);
    sc.cwd = static_cast<float>(1.0 - a->lr * a->weight_decay);
    sc.b1 = static_cast<float>(a->beta1);
    sc.c1 = static_cast<float>(1.0 - a->beta1);
    sc.b2 = static_cast<float>(a->beta2);
    sc.c2 = static_cast<float>(1.0 - a->beta2);
    sc.bc1 = static_cast<float>(1.0 - std::pow(a->beta1, t));
    sc.bc2 = static_cast<float>(1.0 - std::pow(a->beta2, t));
    sc.lr = static_cast<float>(a->lr);
    sc.eps = static_cast<float>(a->eps);
    // 1 - beta^t >= 1 - beta >= 2^-53 for beta in [0, 1): positive and normal
    sc.inv_bc2s = 0x1p64 / static_cast<double>(sc.bc2);
    {
        // 1 / bc1 correctly rounded to fp32: the neighbour of the double
        // quotient rounded to float with the smallest residual |r bc1 - 1|
        // (exact in double: a product of two floats)
        float r = static_cast<float>(1.0 / static_cast<double>(sc.bc1));
        const float cand[3] = {std::nextafter(r, 0.0f), r, std::nextafter(r, INFINITY)};
        double best = INFINITY;
        for (float c : cand) {
            const double e = std::fabs(static_cast<double>(c) * static_cast<double>(sc.bc1) - 1.0);
            if (e < best) { best = e; r = c; }
        }
        sc.rbc1 = r;
    }
    sc.unit_bc = (sc.bc1 == 1.0f ? 1 : 0) | (sc.bc2 == 1.0f ? 2 : 0);
    sc.lr2 = sc.lr * 0x1p32f;
    sc.eps2 = sc.eps * 0x1p32f;
    sc.kv = static_cast<float>(255.0 * std::sqrt(static_cast<double>(sc.bc2)) * 0x1p-32);
    // The kernel's short route (step_finish) is exact under these bounds.
    // Its sqrt returns sqrt(vhat) 2^32, except a value below 2^-31 (not the
    // exact root) for a subnormal or zero vhat, which vanishes next to eps2
    // (half an ulp of eps2 is at least 2^-30 while eps >= 2^-38).  The short
    // division needs denominators in [2^-100, 2^100] (eps2 >= 2^-6 and
    // sqrt(vhat) 2^32 < 2^64) and numerators of at most 2^100 eps2 and, when
    // nonzero, at least 2^-61 (the lane checks both).  mhat = m1 / bc1 comes
    // from div_markstein with rbc1, exact for m1 = 0 and for 2^-102 <= |m1|
    // <= 2^100 bc1 (bc1 is in [2^-53, 1]); |m1| <= m1_max <= 2^99 bc1 covers
    // the upper end.  A nonzero |m1| below 2^-102 gives |mhat| < 2^-101 / bc1
    // (up to a few units of 2^-149), so with lr <= 2^6 bc1 its numerator
    // lr2 mhat stays below 2^-61 and the lane takes the generic route; with
    // lr >= 2^-32 (lr2 >= 1) no nonzero mhat gives a zero numerator, and
    // lr = 0 gives the zero numerator of the exact evaluation.
    sc.fast = (sc.eps >= 0x1p-38f && sc.eps <= 0x1p60f &&
               (sc.lr == 0.0f ||
                (sc.lr >= 0x1p-32f && static_cast<double>(sc.lr) <= 0x1p6 * static_cast<double>(sc.bc1))))
                  ? 1 : 0;
    // vhat = v1 / bc2 < 2^63  <=  v1 < 2^63 bc2 (rounded down to fp32)
    {
        float vb = static_cast<float>(0x1p63 * static_cast<double>(sc.bc2));
        if (static_cast<double>(vb) > 0x1p63 * static_cast<double>(sc.bc2))
            vb = std::nextafter(vb, 0.0f);
        uint32_t bits;
        std::memcpy(&bits, &vb, 4);
        sc.v1_bound = bits;
    }
    // |lr2 mhat| <= 2^100 eps2 holds when lr2 |m1| / bc1 (1 + 2^-20) does;
    // |m1| <= 2^99 bc1 keeps mhat's division in its exact range
    sc.m1_max = sc.lr2 > 0.0f
        ? static_cast<float>(0x1p100 * static_cast<double>(sc.eps2) * static_cast<double>(sc.bc1) /
                             (static_cast<double>(sc.lr2) * (1.0 + 0x1p-20)))
        : INFINITY;
    sc.m1_max = std::fmin(sc.m1_max, static_cast<float>(0x1p99 * static_cast<double>(sc.bc1)));
    {
        const float tmin = 0x1p-61f;
        uint32_t bits;
        std::memcpy(&bits, &tmin, 4);
        sc.num_key = (bits << 1) - 1u;
    }
    return FLASHOPT_OK;
}

flashopt_status sgd_scalars(const flashopt_sgd_args *a, SgdScalars &sc)
{
    if (!a) return FLASHOPT_EINVAL;
    if (a->master_bits != 24 && a->master_bits != 32 && a->master_bits != 0) return FLASHOPT_EINVAL;
    if (a->companded != 0 && a->companded != 1) return FLASHOPT_EINVAL;
    if (a->fp32_states != 0 && a->fp32_states != 1) return FLASHOPT_EINVAL;
    if (a->nesterov != 0 && a->nesterov != 1) return FLASHOPT_EINVAL;
    if (a->step < 1) return FLASHOPT_EINVAL;
    if (!(a->lr >= 0.0) || !std::isfinite(a->lr)) return FLASHOPT_EINVAL;
    if (!(a->momentum > 0.0) || !std::isfinite(a->momentum)) return FLASHOPT_EINVAL;
    if (!std::isfinite(a->dampening) || !std::isfinite(a->weight_decay)) return FLASHOPT_EINVAL;
    if (a->nesterov && a->dampening != 0.0) return FLASHOPT_EINVAL;
    if (a->state_layout != FLASHOPT_STATE_STREAMS && a->state_layout != FLASHOPT_STATE_BLOCKED)
        return FLASHOPT_EINVAL;
    if (a->state_layout == FLASHOPT_STATE_BLOCKED && a->fp32_states) return FLASHOPT_EINVAL;
    sc.blk = state_layout(a->state_layout, a->master_bits, false);
    sc.lr = static_cast<float>(a->lr);
    sc.mu = static_cast<float>(a->momentum);
    sc.cd = static_cast<float>(1.0 - a->dampening);
    sc.wd = static_cast<float>(a->weight_decay);
    sc.has_wd = a->weight_decay != 0.0 ? 1 : 0;
    sc.first = a->step == 1 ? 1 : 0;
    sc.nesterov = a->nesterov;
    return FLASHOPT_OK;
}

// Validation of a step's tensor list; total = its chunks of 1024 elements.
// split: rho is used; quant: scales are used; v: the variance streams are
// used; blocked: the chunk-blocked state layout.
flashopt_status check_list(const flashopt_tensor *tensors, int n_tensors, int master_bits,
                           bool quant, bool v, bool blocked, int64_t &total)
{
    const bool split = master_bits != 0;
    total = 0;
    for (int i = 0; i < n_tensors; ++i) {
        const flashopt_status st = check_tensor(tensors[i], split, quant, v, blocked);
        if (st != FLASHOPT_OK) return st;
        total += (tensors[i].numel + flashopt::kChunkElems - 1) / flashopt::kChunkElems;
        if (total > INT32_MAX) return FLASHOPT_EINVAL;
    }
    return FLASHOPT_OK;
}

// The chunk table of a list: n descriptors, then n + 1 chunk starts (prefix
// sums of the tensors' chunk counts), at `table`.  Returns the total.
int32_t fill_table(const flashopt_tensor *tensors, int n_tensors, void *table)
{
    DevTensor *desc = static_cast<DevTensor *>(table);
    int32_t *start = reinterpret_cast<int32_t *>(desc + n_tensors);
    int32_t acc = 0;
    for (int i = 0; i < n_tensors; ++i) {
        desc[i] = device_descriptor(tensors[i]);
        start[i] = acc;
        acc += static_cast<int32_t>((tensors[i].numel + flashopt::kChunkElems - 1) / flashopt::kChunkElems);
    }
    start[n_tensors] = acc;
    return acc;
}

// Copies `bytes` of host data, which fill(host) writes into a pinned ring
// slot, to device memory `dst` on stream st (the slot is reused once that
// copy has completed).  Returns what fill returned through `out`.
template <typename Fill>
flashopt_status stage_copy(void *dst, size_t bytes, hipStream_t st, Fill &&fill)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FLASHOPT_EHIP;

    std::lock_guard<std::mutex> lock(g_ring_mutex);
    Ring &ring = g_rings[dev];
    Slot &slot = ring.slot[ring.next];
    ring.next = (ring.next + 1) % kRingSlots;
    if (slot.pending) {
        if (hipEventSynchronize(slot.done) != hipSuccess) return FLASHOPT_EHIP;
        slot.pending = false;
    }
    if (!slot.done && hipEventCreateWithFlags(&slot.done, hipEventDisableTiming) != hipSuccess)
        return FLASHOPT_EHIP;
    if (slot.cap < bytes) {
        if (slot.host) (void)hipHostFree(slot.host);
        slot.host = nullptr;
        slot.cap = 0;
        if (hipHostMalloc(&slot.host, bytes, hipHostMallocDefault) != hipSuccess) return FLASHOPT_EHIP;
        slot.cap = bytes;
    }
    fill(slot.host);
    if (hipMemcpyAsync(dst, slot.host, bytes, hipMemcpyHostToDevice, st) != hipSuccess)
        return FLASHOPT_EHIP;
    if (hipEventRecord(slot.done, st) != hipSuccess) return FLASHOPT_EHIP;
    slot.pending = true;
    return FLASHOPT_OK;
}

// Validation of a step's tensor list, then the header (header_bytes of
// `header`, none for 0) and the chunk table staged through the pinned ring
// into the workspace, and launch(d_header, d_desc, d_chunk_start,
// total_chunks, stream).
template <typename Launch>
flashopt_status stage_and_launch(const flashopt_tensor *tensors, int n_tensors, int master_bits,
                                 bool quant, bool v, bool blocked, const void *header,
                                 size_t header_bytes, void *workspace, size_t ws_bytes, void *stream,
                                 Launch &&launch)
{
    int64_t total = 0;
    const flashopt_status cs = check_list(tensors, n_tensors, master_bits, quant, v, blocked, total);
    if (cs != FLASHOPT_OK) return cs;
    if (total == 0) return FLASHOPT_OK;
    const size_t need = staged_bytes(n_tensors, header_bytes);
    if (!workspace || ws_bytes < need) return FLASHOPT_EWORKSPACE;
    if (!aligned(workspace, 16)) return FLASHOPT_EALIGN;

    hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t acc = 0;
    const flashopt_status ss = stage_copy(workspace, need, st, [&](void *host) {
        if (header_bytes) std::memcpy(host, header, header_bytes);
        acc = fill_table(tensors, n_tensors, static_cast<unsigned char *>(host) + header_bytes);
    });
    if (ss != FLASHOPT_OK) return ss;

    const unsigned char *base = static_cast<const unsigned char *>(workspace);
    const DevTensor *d_desc = reinterpret_cast<const DevTensor *>(base + header_bytes);
    const int32_t *d_start = reinterpret_cast<const int32_t *>(d_desc + n_tensors);
    return hip_status(launch(base, d_desc, d_start, acc, st));
}

// Plans (the capture-safe list steps): the tables and the scalar block of
// a list staged once into a caller's device buffer, the scalar block
// rewritten per step, and launches that only enqueue the kernel.

// Validation of a plan's list, then its scalar block and tables staged into
// `plan`; n_tensors and total_chunks of the plan go to info.
template <typename Sc, typename Info>
flashopt_status make_plan(const flashopt_tensor *tensors, int n_tensors, int master_bits, bool quant,
                          bool v, bool blocked, const Sc &sc, void *plan, size_t plan_bytes,
                          Info &info, void *stream)
{
    int64_t total = 0;
    const flashopt_status cs = check_list(tensors, n_tensors, master_bits, quant, v, blocked, total);
    if (cs != FLASHOPT_OK) return cs;
    const size_t need = staged_bytes(n_tensors, kHeader);
    if (need > 0 && (!plan || plan_bytes < need)) return FLASHOPT_EWORKSPACE;
    if (need > 0 && !aligned(plan, 16)) return FLASHOPT_EALIGN;
    if (need > 0) {
        const flashopt_status ss = stage_copy(plan, need, static_cast<hipStream_t>(stream), [&](void *host) {
            fill_scalars(sc, host);
            (void)fill_table(tensors, n_tensors, static_cast<unsigned char *>(host) + kHeader);
        });
        if (ss != FLASHOPT_OK) return ss;
    }
    info.n_tensors = n_tensors;
    info.total_chunks = static_cast<int32_t>(total);
    return FLASHOPT_OK;
}

// A new scalar block for a plan of n_tensors tensors.
template <typename Sc>
flashopt_status plan_scalars(int n_tensors, const Sc &sc, void *plan, void *stream)
{
    if (n_tensors <= 0) return n_tensors == 0 ? FLASHOPT_OK : FLASHOPT_EINVAL;
    if (!plan) return FLASHOPT_EWORKSPACE;
    if (!aligned(plan, 16)) return FLASHOPT_EALIGN;
    return stage_copy(plan, kHeader, static_cast<hipStream_t>(stream),
                      [&](void *host) { fill_scalars(sc, host); });
}

// The device pointers of a plan: scalar block, descriptors, chunk starts.
struct PlanPtrs {
    const void *scalars;
    const DevTensor *desc;
    const int32_t *start;
};

PlanPtrs plan_ptrs(const void *plan, int n_tensors)
{
    const unsigned char *base = static_cast<const unsigned char *>(plan);
    const DevTensor *d = reinterpret_cast<const DevTensor *>(base + kHeader);
    return PlanPtrs{base, d, reinterpret_cast<const int32_t *>(d + n_tensors)};
}

bool same_variant(const flashopt_adamw_args &a, const flashopt_adamw_plan_info &info)
{
    return info.master_bits == a.master_bits && info.companded == a.companded &&
           info.fp32_states == a.fp32_states && info.param_fp32 == a.param_fp32 &&
           info.state_layout == a.state_layout;
}

bool same_variant(const flashopt_sgd_args &a, const flashopt_sgd_plan_info &info)
{
    return info.master_bits == a.master_bits && info.companded == a.companded &&
           info.fp32_states == a.fp32_states && info.state_layout == a.state_layout;
}

// The launch-time checks shared by both plan kinds: counts, then the buffer.
flashopt_status plan_launch_checks(int32_t n_tensors, int32_t total_chunks, const void *plan)
{
    if (n_tensors < 0 || total_chunks < 0) return FLASHOPT_EINVAL;
    if (total_chunks == 0) return FLASHOPT_OK;
    if (n_tensors == 0) return FLASHOPT_EINVAL;
    if (!plan) return FLASHOPT_EWORKSPACE;
    if (!aligned(plan, 16)) return FLASHOPT_EALIGN;
    return FLASHOPT_OK;
}

bool valid_variant(int master_bits, int companded, int fp32_states)
{
    return (master_bits == 24 || master_bits == 32 || master_bits == 0) &&
           (companded == 0 || companded == 1) && (fp32_states == 0 || fp32_states == 1);
}

// A state layout, and whether the storage variant allows it (the blocked
// layout holds quantized states only).
bool valid_layout(int layout, int fp32_states)
{
    return layout == FLASHOPT_STATE_STREAMS || (layout == FLASHOPT_STATE_BLOCKED && fp32_states == 0);
}

// Host image of the allocation-free step's scalar block and chunk table:
// built under the mutex and copied (pageable hipMemcpyAsync, which has
// consumed the buffer when it returns) into the device scratch array.
std::mutex g_noalloc_mutex;
alignas(64) unsigned char g_noalloc_table[flashopt::kScratchBytes];

}  // namespace

extern "C" {

int flashopt_abi_version(void) { return FLASHOPT_ABI_VERSION; }

size_t flashopt_blocked_state_bytes(int64_t numel, int master_bits, int with_variance)
{
    if (numel <= 0 || (master_bits != 24 && master_bits != 32 && master_bits != 0)) return 0;
    const flashopt::StateLayout L = state_layout(FLASHOPT_STATE_BLOCKED, master_bits, with_variance != 0);
    const int64_t chunks = (numel + flashopt::kChunkElems - 1) / flashopt::kChunkElems;
    return static_cast<size_t>(chunks) * L.bytes;
}

const char *flashopt_status_str(flashopt_status s)
{
    switch (s) {
    case FLASHOPT_OK: return "FLASHOPT_OK";
    case FLASHOPT_EINVAL: return "FLASHOPT_EINVAL: invalid argument";
    case FLASHOPT_EALIGN: return "FLASHOPT_EALIGN: buffer not aligned (16 B streams, 2 B scales)";
    case FLASHOPT_EWORKSPACE: return "FLASHOPT_EWORKSPACE: workspace missing or too small";
    case FLASHOPT_EHIP: return "FLASHOPT_EHIP: HIP runtime error on enqueue";
    }
    return "FLASHOPT_UNKNOWN_STATUS";
}

flashopt_status flashopt_quantize(const float *x, int64_t n, unsigned spec, void *codes,
                                  uint16_t *scales, void *stream)
{
    flashopt_status st = check_codec(x, n, spec, codes, scales);
    if (st != FLASHOPT_OK || n == 0) return st;
    return hip_status(flashopt::launch_quantize(x, n, spec, codes, scales,
                                                static_cast<hipStream_t>(stream)));
}

flashopt_status flashopt_dequantize(const void *codes, const uint16_t *scales, int64_t n,
                                    unsigned spec, float *out, void *stream)
{
    flashopt_status st = check_codec(out, n, spec, codes, scales);
    if (st != FLASHOPT_OK || n == 0) return st;
    return hip_status(flashopt::launch_dequantize(codes, scales, n, spec, out,
                                                  static_cast<hipStream_t>(stream)));
}

flashopt_status flashopt_split(const float *master, int64_t n, int master_bits,
                               uint16_t *param_bf16, void *rho, void *stream)
{
    flashopt_status st = check_split(master, n, master_bits, param_bf16, rho);
    if (st != FLASHOPT_OK || n == 0) return st;
    return hip_status(flashopt::launch_split(master, n, master_bits, param_bf16, rho,
                                             static_cast<hipStream_t>(stream)));
}

flashopt_status flashopt_reconstruct(const uint16_t *param_bf16, const void *rho, int64_t n,
                                     int master_bits, float *master, void *stream)
{
    flashopt_status st = check_split(master, n, master_bits, param_bf16, rho);
    if (st != FLASHOPT_OK || n == 0) return st;
    return hip_status(flashopt::launch_reconstruct(param_bf16, rho, n, master_bits, master,
                                                   static_cast<hipStream_t>(stream)));
}

size_t flashopt_adamw_workspace_bytes(const flashopt_tensor *tensors, int n_tensors)
{
    (void)tensors;
    return staged_bytes(n_tensors, kHeader);
}

flashopt_status flashopt_adamw_step(const flashopt_tensor *tensors, int n_tensors,
                                    const flashopt_adamw_args *a, void *workspace,
                                    size_t ws_bytes, void *stream)
{
    if (n_tensors < 0 || (n_tensors > 0 && !tensors)) return FLASHOPT_EINVAL;
    StepScalars sc;
    const flashopt_status hs = adamw_scalars(a, sc);
    if (hs != FLASHOPT_OK) return hs;
    const int states = states_of(a->fp32_states, a->companded);
    alignas(16) unsigned char header[kHeader];
    fill_scalars(sc, header);
    return stage_and_launch(tensors, n_tensors, a->master_bits, a->fp32_states == 0, true,
                            a->state_layout == FLASHOPT_STATE_BLOCKED, header, kHeader, workspace,
                            ws_bytes, stream,
                            [&](const unsigned char *h, const DevTensor *d, const int32_t *cs,
                                int32_t total, hipStream_t st) {
                                return flashopt::launch_adamw_step(
                                    reinterpret_cast<const StepScalars *>(h), d, cs, n_tensors,
                                    total, kernel_format(*a), states, st);
                            });
}

flashopt_status flashopt_adamw_step_tensor(const flashopt_tensor *tensor,
                                           const flashopt_adamw_args *a, void *stream)
{
    if (!tensor) return FLASHOPT_EINVAL;
    StepScalars sc;
    const flashopt_status hs = adamw_scalars(a, sc);
    if (hs != FLASHOPT_OK) return hs;
    const flashopt_status ts = check_tensor(*tensor, a->master_bits != 0, a->fp32_states == 0, true,
                                            a->state_layout == FLASHOPT_STATE_BLOCKED);
    if (ts != FLASHOPT_OK || tensor->numel == 0) return ts;
    return hip_status(flashopt::launch_adamw_tensor(device_descriptor(*tensor), sc, kernel_format(*a),
                                                    states_of(a->fp32_states, a->companded),
                                                    static_cast<hipStream_t>(stream)));
}

flashopt_status flashopt_adamw_step_noalloc(const flashopt_tensor *tensors, int n_tensors,
                                            const flashopt_adamw_args *a, void *stream)
{
    if (n_tensors < 0 || (n_tensors > 0 && !tensors)) return FLASHOPT_EINVAL;
    if (n_tensors > flashopt::kScratchTensors) return FLASHOPT_EWORKSPACE;
    StepScalars sc;
    const flashopt_status hs = adamw_scalars(a, sc);
    if (hs != FLASHOPT_OK) return hs;
    int64_t total = 0;
    const flashopt_status cs = check_list(tensors, n_tensors, a->master_bits, a->fp32_states == 0,
                                          true, a->state_layout == FLASHOPT_STATE_BLOCKED, total);
    if (cs != FLASHOPT_OK || total == 0) return cs;
    void *scratch = nullptr;
    if (flashopt::scratch_address(&scratch) != hipSuccess) return FLASHOPT_EHIP;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t acc = 0;
    {
        std::lock_guard<std::mutex> lock(g_noalloc_mutex);
        fill_scalars(sc, g_noalloc_table);
        acc = fill_table(tensors, n_tensors, g_noalloc_table + kHeader);
        if (hipMemcpyAsync(scratch, g_noalloc_table, staged_bytes(n_tensors, kHeader),
                           hipMemcpyHostToDevice, st) != hipSuccess)
            return FLASHOPT_EHIP;
    }
    const unsigned char *base = static_cast<const unsigned char *>(scratch);
    const DevTensor *d_desc = reinterpret_cast<const DevTensor *>(base + kHeader);
    const int32_t *d_start = reinterpret_cast<const int32_t *>(d_desc + n_tensors);
    return hip_status(flashopt::launch_adamw_step(reinterpret_cast<const StepScalars *>(base), d_desc,
                                                  d_start, n_tensors, acc, kernel_format(*a),
                                                  states_of(a->fp32_states, a->companded), st));
}

size_t flashopt_adamw_plan_bytes(int n_tensors)
{
    return staged_bytes(n_tensors, kHeader);
}

flashopt_status flashopt_adamw_plan(const flashopt_tensor *tensors, int n_tensors,
                                    const flashopt_adamw_args *a, void *plan, size_t plan_bytes,
                                    flashopt_adamw_plan_info *info, void *stream)
{
    if (!info || n_tensors < 0 || (n_tensors > 0 && !tensors)) return FLASHOPT_EINVAL;
    StepScalars sc;
    const flashopt_status hs = adamw_scalars(a, sc);
    if (hs != FLASHOPT_OK) return hs;
    flashopt_adamw_plan_info out{};
    out.master_bits = a->master_bits;
    out.companded = a->companded;
    out.fp32_states = a->fp32_states;
    out.param_fp32 = a->param_fp32;
    out.state_layout = a->state_layout;
    const flashopt_status ps = make_plan(tensors, n_tensors, a->master_bits, a->fp32_states == 0, true,
                                         a->state_layout == FLASHOPT_STATE_BLOCKED, sc, plan,
                                         plan_bytes, out, stream);
    if (ps == FLASHOPT_OK) *info = out;
    return ps;
}

flashopt_status flashopt_adamw_plan_set_step(const flashopt_adamw_plan_info *info,
                                             const flashopt_adamw_args *a, void *plan, void *stream)
{
    if (!info || !a || !same_variant(*a, *info)) return FLASHOPT_EINVAL;
    StepScalars sc;
    const flashopt_status hs = adamw_scalars(a, sc);
    if (hs != FLASHOPT_OK) return hs;
    return plan_scalars(info->n_tensors, sc, plan, stream);
}

flashopt_status flashopt_adamw_plan_launch(const flashopt_adamw_plan_info *info, const void *plan,
                                           void *stream)
{
    if (!info) return FLASHOPT_EINVAL;
    if (!valid_variant(info->master_bits, info->companded, info->fp32_states) ||
        (info->param_fp32 != 0 && info->param_fp32 != 1) || (info->param_fp32 && info->master_bits != 0) ||
        !valid_layout(info->state_layout, info->fp32_states))
        return FLASHOPT_EINVAL;
    const flashopt_status lc = plan_launch_checks(info->n_tensors, info->total_chunks, plan);
    if (lc != FLASHOPT_OK || info->total_chunks == 0) return lc;
    flashopt_adamw_args a{};
    a.master_bits = info->master_bits;
    a.param_fp32 = info->param_fp32;
    const PlanPtrs p = plan_ptrs(plan, info->n_tensors);
    return hip_status(flashopt::launch_adamw_step(static_cast<const StepScalars *>(p.scalars), p.desc,
                                                  p.start, info->n_tensors, info->total_chunks,
                                                  kernel_format(a),
                                                  states_of(info->fp32_states, info->companded),
                                                  static_cast<hipStream_t>(stream)));
}

size_t flashopt_sgd_workspace_bytes(const flashopt_tensor *tensors, int n_tensors)
{
    (void)tensors;
    return staged_bytes(n_tensors, kHeader);
}

flashopt_status flashopt_sgd_step(const flashopt_tensor *tensors, int n_tensors,
                                  const flashopt_sgd_args *a, void *workspace,
                                  size_t ws_bytes, void *stream)
{
    if (n_tensors < 0 || (n_tensors > 0 && !tensors)) return FLASHOPT_EINVAL;
    SgdScalars sc;
    const flashopt_status hs = sgd_scalars(a, sc);
    if (hs != FLASHOPT_OK) return hs;
    const int states = states_of(a->fp32_states, a->companded);
    alignas(16) unsigned char header[kHeader];
    fill_scalars(sc, header);
    return stage_and_launch(tensors, n_tensors, a->master_bits, a->fp32_states == 0, false,
                            a->state_layout == FLASHOPT_STATE_BLOCKED, header, kHeader, workspace,
                            ws_bytes, stream,
                            [&](const unsigned char *h, const DevTensor *d, const int32_t *cs,
                                int32_t total, hipStream_t st) {
                                return flashopt::launch_sgd_step(
                                    reinterpret_cast<const SgdScalars *>(h), d, cs, n_tensors, total,
                                    a->master_bits, states, st);
                            });
}

size_t flashopt_sgd_plan_bytes(int n_tensors)
{
    return staged_bytes(n_tensors, kHeader);
}

flashopt_status flashopt_sgd_plan(const flashopt_tensor *tensors, int n_tensors,
                                  const flashopt_sgd_args *a, void *plan, size_t plan_bytes,
                                  flashopt_sgd_plan_info *info, void *stream)
{
    if (!info || n_tensors < 0 || (n_tensors > 0 && !tensors)) return FLASHOPT_EINVAL;
    SgdScalars sc;
    const flashopt_status hs = sgd_scalars(a, sc);
    if (hs != FLASHOPT_OK) return hs;
    flashopt_sgd_plan_info out{};
    out.master_bits = a->master_bits;
    out.companded = a->companded;
    out.fp32_states = a->fp32_states;
    out.state_layout = a->state_layout;
    const flashopt_status ps = make_plan(tensors, n_tensors, a->master_bits, a->fp32_states == 0, false,
                                         a->state_layout == FLASHOPT_STATE_BLOCKED, sc, plan,
                                         plan_bytes, out, stream);
    if (ps == FLASHOPT_OK) *info = out;
    return ps;
}

flashopt_status flashopt_sgd_plan_set_step(const flashopt_sgd_plan_info *info,
                                           const flashopt_sgd_args *a, void *plan, void *stream)
{
    if (!info || !a || !same_variant(*a, *info)) return FLASHOPT_EINVAL;
    SgdScalars sc;
    const flashopt_status hs = sgd_scalars(a, sc);
    if (hs != FLASHOPT_OK) return hs;
    return plan_scalars(info->n_tensors, sc, plan, stream);
}

flashopt_status flashopt_sgd_plan_launch(const flashopt_sgd_plan_info *info, const void *plan,
                                         void *stream)
{
    if (!info) return FLASHOPT_EINVAL;
    if (!valid_variant(info->master_bits, info->companded, info->fp32_states) ||
        !valid_layout(info->state_layout, info->fp32_states))
        return FLASHOPT_EINVAL;
    const flashopt_status lc = plan_launch_checks(info->n_tensors, info->total_chunks, plan);
    if (lc != FLASHOPT_OK || info->total_chunks == 0) return lc;
    const PlanPtrs p = plan_ptrs(plan, info->n_tensors);
    return hip_status(flashopt::launch_sgd_step(static_cast<const SgdScalars *>(p.scalars), p.desc,
                                                p.start, info->n_tensors, info->total_chunks,
                                                info->master_bits,
                                                states_of(info->fp32_states, info->companded),
                                                static_cast<hipStream_t>(stream)));
}

flashopt_status flashopt_sgd_step_tensor(const flashopt_tensor *tensor,
                                         const flashopt_sgd_args *a, void *stream)
{
    if (!tensor) return FLASHOPT_EINVAL;
    SgdScalars sc;
    const flashopt_status hs = sgd_scalars(a, sc);
    if (hs != FLASHOPT_OK) return hs;
    const flashopt_status ts = check_tensor(*tensor, a->master_bits != 0, a->fp32_states == 0, false,
                                            a->state_layout == FLASHOPT_STATE_BLOCKED);
    if (ts != FLASHOPT_OK || tensor->numel == 0) return ts;
    return hip_status(flashopt::launch_sgd_tensor(device_descriptor(*tensor), sc, a->master_bits,
                                                  states_of(a->fp32_states, a->companded),
                                                  static_cast<hipStream_t>(stream)));
}

}  // extern "C"
