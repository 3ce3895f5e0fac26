// msel_api.cpp -- the extern "C" entry points declared in include/msel.h.
//
// Every entry point first validates its arguments on the host (no HIP call, no device memory
// touched) and only then enqueues kernels on the caller's stream.  The library never
// allocates and never synchronizes; its only state is the ring-wait timeout count and limit
// (msel_ring_timeouts, msel_set_ring_spin_limit), whose reader synchronizes.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <mutex>

#include "msel.h"  // include/ is on the include path
#include "msel_kernels.hpp"

static_assert(MSEL_MAX_DSTATE == msel::kMaxN, "the kernels' state limit is the boundary's");

namespace {

constexpr int64_t kMaxSeq = MSEL_MAX_SEQLEN;
constexpr int64_t kMaxRows = int64_t(1) << 30;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

msel_status check_common(const msel_scan_args* a) {
    if (a == nullptr) return MSEL_ERR_NULL;
    if (a->abi_version != MSEL_ABI_VERSION || a->reserved != 0) return MSEL_ERR_VERSION;
    if (a->batch < 1 || a->dim < 1 || a->dstate < 1 || a->seqlen < 1) return MSEL_ERR_SHAPE;
    if (static_cast<int64_t>(a->batch) * a->dim > kMaxRows || a->seqlen > kMaxSeq)
        return MSEL_ERR_SHAPE;
    if (a->dtype != MSEL_F32 && a->dtype != MSEL_BF16) return MSEL_ERR_DTYPE;
    if (a->delta_softplus != 0 && a->delta_softplus != 1) return MSEL_ERR_DTYPE;
    if (a->dstate > MSEL_MAX_DSTATE) return MSEL_ERR_UNSUPPORTED;
    if (a->u == nullptr || a->delta == nullptr || a->B == nullptr || a->A == nullptr)
        return MSEL_ERR_NULL;
    const void* act[] = {a->u, a->delta, a->B, a->C, a->z};
    for (const void* p : act)
        if (p != nullptr && !aligned(p, 16)) return MSEL_ERR_ALIGN;
    const void* f32[] = {a->A, a->D, a->delta_bias, a->h0, a->final_state, a->chunk_states};
    for (const void* p : f32)
        if (p != nullptr && !aligned(p, 4)) return MSEL_ERR_ALIGN;
    return MSEL_OK;
}

bool same_as_input(const msel_scan_args* a, const void* o) {
    if (o == nullptr) return false;
    const void* in[] = {a->u, a->delta, a->B, a->C, a->z, a->A, a->D, a->delta_bias, a->h0};
    for (const void* p : in)
        if (p != nullptr && p == o) return true;
    return false;
}

// final_state may be h0 itself (the state updated in place, as a decode cache is): each
// wavefront reads its channels' h0 before it writes their final state.
bool final_state_aliases(const msel_scan_args* a) {
    return a->final_state != a->h0 && same_as_input(a, a->final_state);
}

msel::ScanParams to_params(const msel_scan_args* a) {
    msel::ScanParams p;
    p.B = a->batch;
    p.D = a->dim;
    p.N = a->dstate;
    p.L = a->seqlen;
    p.nchunks = msel_num_chunks(a->seqlen);
    p.softplus = a->delta_softplus;
    p.u = a->u;
    p.delta = a->delta;
    p.Bm = a->B;
    p.Cm = a->C;
    p.z = a->z;
    p.A = a->A;
    p.Dv = a->D;
    p.bias = a->delta_bias;
    p.h0 = a->h0;
    p.out = a->out;
    p.final_state = a->final_state;
    p.chunk_states = a->chunk_states;
    return p;
}

msel_status hip_status(hipError_t e) { return e == hipSuccess ? MSEL_OK : MSEL_ERR_HIP; }

// ---- the short causal convolution ------------------------------------------------------

size_t elem_bytes(int32_t dtype) { return dtype == MSEL_BF16 ? 2 : 4; }

msel_status check_conv(const msel_conv_args* a) {
    if (a == nullptr) return MSEL_ERR_NULL;
    if (a->abi_version != MSEL_ABI_VERSION || a->reserved != 0) return MSEL_ERR_VERSION;
    if (a->batch < 1 || a->dim < 1 || a->seqlen < 1 || a->width < 1) return MSEL_ERR_SHAPE;
    if (static_cast<int64_t>(a->batch) * a->dim > kMaxRows || a->seqlen > kMaxSeq)
        return MSEL_ERR_SHAPE;
    if (a->dtype != MSEL_F32 && a->dtype != MSEL_BF16) return MSEL_ERR_DTYPE;
    if (a->activation != 0 && a->activation != 1) return MSEL_ERR_DTYPE;
    if (a->width > MSEL_MAX_CONV_WIDTH) return MSEL_ERR_UNSUPPORTED;
    if (msel::conv_waves(static_cast<int64_t>(a->batch) * a->dim, a->seqlen,
                         a->dtype == MSEL_BF16) > msel::kMaxConvWaves)
        return MSEL_ERR_SHAPE;
    if (a->x == nullptr || a->weight == nullptr) return MSEL_ERR_NULL;
    if (!aligned(a->x, 16)) return MSEL_ERR_ALIGN;
    if (!aligned(a->weight, 4) || (a->bias != nullptr && !aligned(a->bias, 4)))
        return MSEL_ERR_ALIGN;
    if (a->width > 1 && a->state_in != nullptr && !aligned(a->state_in, elem_bytes(a->dtype)))
        return MSEL_ERR_ALIGN;
    return MSEL_OK;
}

bool conv_input(const msel_conv_args* a, const void* o) {
    if (o == nullptr) return false;
    const void* in[] = {a->x, a->weight, a->bias, a->state_in};
    for (const void* p : in)
        if (p != nullptr && p == o) return true;
    return false;
}

msel::ConvParams to_conv_params(const msel_conv_args* a) {
    msel::ConvParams p = {};
    p.rows = static_cast<int64_t>(a->batch) * a->dim;
    p.D = a->dim;
    p.L = a->seqlen;
    p.W = a->width;
    p.silu = a->activation;
    p.x = a->x;
    p.w = a->weight;
    p.bias = a->bias;
    p.state_in = a->width > 1 ? a->state_in : nullptr;
    return p;
}

// Bytes of one set of chunk states, rounded up as the backward's workspace pieces are.
size_t states_bytes_aligned(const msel_scan_args* a) {
    const size_t s = static_cast<size_t>(a->batch) * a->dim * msel_num_chunks(a->seqlen) *
                     a->dstate * sizeof(float);
    return (s + 255) & ~static_cast<size_t>(255);
}

// The backward's launches after validation: zero-fills, then summary, link and gradient
// kernels (the trapezoidal variant when `tr` is given; with no chunk states given, its
// chunk-carry pass rebuilds them first).
msel_status run_bwd(const msel_scan_args* a, const msel_scan_grads* g, const msel_trap_args* tr,
                    const msel_trap_grads* tg, void* workspace, size_t workspace_bytes,
                    hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
    const bool bf16 = a->dtype == MSEL_BF16;
    msel::ScanParams p = to_params(a);
    if (tr != nullptr) {
        p.lam = tr->lambda;
        p.u_prev = tr->u_prev;
        p.B_prev = tr->B_prev;
    }
    const size_t DN = static_cast<size_t>(a->dim) * a->dstate;
    const size_t BNL = static_cast<size_t>(a->batch) * a->dstate * a->seqlen;
    float* dB_prev = tg != nullptr ? tg->dB_prev : nullptr;
    const msel::FillList fill = {{g->dA, g->dB, g->dC, g->dD, g->ddelta_bias, dB_prev},
                                 {DN, BNL, BNL, static_cast<size_t>(a->dim),
                                  static_cast<size_t>(a->dim),
                                  static_cast<size_t>(a->batch) * a->dstate}};
    msel::GradParams gp;
    gp.dout = g->dout;
    gp.du = g->du;
    gp.ddelta = g->ddelta;
    gp.dz = g->dz;
    gp.dA = g->dA;
    gp.dB = g->dB;
    gp.dC = g->dC;
    gp.dD = g->dD;
    gp.dbias = g->ddelta_bias;
    gp.dh0 = g->dh0;
    if (tg != nullptr) {
        gp.dlam = tg->dlambda;
        gp.du_prev = tg->du_prev;
        gp.dB_prev = tg->dB_prev;
    }
    const float* states = a->chunk_states;
    if (tr != nullptr && states == nullptr) {
        // the trapezoidal forward's chunk states, rebuilt by its chunk-carry pass into the
        // front of the workspace; the rest is laid out as with the states given
        float* H = static_cast<float*>(workspace);
        msel::ScanParams pc = p;
        pc.chunk_states = H;
        pc.final_state = nullptr;
        if (msel::launch_chunk_carry(pc, bf16, false, stream) != hipSuccess) return MSEL_ERR_HIP;
        states = H;
        workspace = static_cast<char*>(workspace) + states_bytes_aligned(a);
        workspace_bytes -= states_bytes_aligned(a);
    }
    return hip_status(msel::launch_scan_bwd(p, gp, states, workspace, workspace_bytes, bf16,
                                            fill, stream, ev_begin, ev_end));
}

}  // namespace

extern "C" {

int32_t msel_abi_version(void) { return MSEL_ABI_VERSION; }

int32_t msel_chunk_len(void) { return msel::kChunk; }

int32_t msel_num_chunks(int32_t seqlen) {
    if (seqlen < 1) return 0;
    return static_cast<int32_t>((static_cast<int64_t>(seqlen) + msel::kChunk - 1) / msel::kChunk);
}

const char* msel_status_string(msel_status s) {
    switch (s) {
        case MSEL_OK: return "MSEL_OK";
        case MSEL_ERR_NULL: return "MSEL_ERR_NULL: a required pointer is NULL";
        case MSEL_ERR_SHAPE: return "MSEL_ERR_SHAPE: a size is out of range";
        case MSEL_ERR_DTYPE: return "MSEL_ERR_DTYPE: unknown dtype or softplus flag";
        case MSEL_ERR_ALIGN: return "MSEL_ERR_ALIGN: a pointer is not aligned";
        case MSEL_ERR_UNSUPPORTED: return "MSEL_ERR_UNSUPPORTED: dstate above MSEL_MAX_DSTATE";
        case MSEL_ERR_WORKSPACE: return "MSEL_ERR_WORKSPACE: workspace missing or too small";
        case MSEL_ERR_ALIAS: return "MSEL_ERR_ALIAS: an output aliases an input";
        case MSEL_ERR_HIP: return "MSEL_ERR_HIP: the HIP runtime reported an error";
        case MSEL_ERR_VERSION: return "MSEL_ERR_VERSION: ABI version or reserved field mismatch";
        case MSEL_ERR_TOO_LARGE:
            return "MSEL_ERR_TOO_LARGE: the problem needs more than the library's static scratch "
                   "(MSEL_NOALLOC_SCRATCH_BYTES)";
    }
    return "MSEL_ERR_UNKNOWN";
}

msel_status msel_validate_fwd(const msel_scan_args* a) {
    msel_status s = check_common(a);
    if (s != MSEL_OK) return s;
    if (a->C == nullptr || a->out == nullptr) return MSEL_ERR_NULL;
    if (!aligned(a->out, 16)) return MSEL_ERR_ALIGN;
    if (same_as_input(a, a->out) || final_state_aliases(a) || same_as_input(a, a->chunk_states))
        return MSEL_ERR_ALIAS;
    if (a->out == a->final_state || a->out == a->chunk_states ||
        (a->chunk_states != nullptr && a->chunk_states == a->final_state))
        return MSEL_ERR_ALIAS;
    return MSEL_OK;
}

msel_status msel_validate_trap_fwd(const msel_scan_args* a, const msel_trap_args* tr) {
    msel_status s = msel_validate_fwd(a);
    if (s != MSEL_OK) return s;
    if (tr == nullptr || tr->lambda == nullptr) return MSEL_ERR_NULL;
    if (!aligned(tr->lambda, 16)) return MSEL_ERR_ALIGN;
    const size_t e = a->dtype == MSEL_BF16 ? 2 : 4;
    if ((tr->u_prev != nullptr && !aligned(tr->u_prev, e)) ||
        (tr->B_prev != nullptr && !aligned(tr->B_prev, e)))
        return MSEL_ERR_ALIGN;
    const void* outs[] = {a->out, a->final_state, a->chunk_states};
    for (const void* o : outs)
        if (o != nullptr && (o == tr->lambda || o == tr->u_prev || o == tr->B_prev))
            return MSEL_ERR_ALIAS;
    return MSEL_OK;
}

msel_status msel_validate_complex_fwd(const msel_scan_args* a) {
    msel_status s = msel_validate_fwd(a);
    if (s != MSEL_OK) return s;
    if (a->dstate % 2 != 0) return MSEL_ERR_SHAPE;  // states come in (Re, Im) pairs
    return MSEL_OK;
}

msel_status msel_validate_chunk_carry(const msel_scan_args* a) {
    msel_status s = check_common(a);
    if (s != MSEL_OK) return s;
    if (a->chunk_states == nullptr) return MSEL_ERR_NULL;
    if (same_as_input(a, a->chunk_states) || final_state_aliases(a) ||
        a->chunk_states == a->final_state)
        return MSEL_ERR_ALIAS;
    return MSEL_OK;
}

size_t msel_scan_bwd_workspace_bytes(const msel_scan_args* a) {
    if (check_common(a) != MSEL_OK) return 0;
    return msel::bwd_workspace_bytes(a->batch, a->dim, a->dstate, a->seqlen,
                                     a->chunk_states == nullptr);
}

}  // extern "C"

namespace {

// The backward's checks that do not involve the workspace.
msel_status check_bwd(const msel_scan_args* a, const msel_scan_grads* g) {
    msel_status s = check_common(a);
    if (s != MSEL_OK) return s;
    if (a->C == nullptr || g == nullptr || g->dout == nullptr || g->du == nullptr ||
        g->ddelta == nullptr)
        return MSEL_ERR_NULL;
    if (a->z != nullptr && g->dz == nullptr) return MSEL_ERR_NULL;
    const void* act[] = {g->dout, g->du, g->ddelta, g->dz};
    for (const void* p : act)
        if (p != nullptr && !aligned(p, 16)) return MSEL_ERR_ALIGN;
    const void* f32[] = {g->dA, g->dB, g->dC, g->dD, g->ddelta_bias, g->dh0};
    for (const void* p : f32)
        if (p != nullptr && !aligned(p, 4)) return MSEL_ERR_ALIGN;
    const void* outs[] = {g->du, g->ddelta, g->dz, g->dA, g->dB, g->dC, g->dD, g->ddelta_bias,
                          g->dh0};
    for (const void* o : outs)
        if (same_as_input(a, o) || (o != nullptr && (o == g->dout || o == a->chunk_states)))
            return MSEL_ERR_ALIAS;
    return MSEL_OK;
}

// ---- the backward without a workspace argument ------------------------------------------
//
// For callers that cannot allocate: the workspace is a file-scope device array of fixed size.
// In host code `scratch` only names the symbol; its device address, one per device, comes
// from hipGetSymbolAddress on the entry point's first call on that device.
constexpr size_t kScratchBytes = MSEL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch`, or null if the device cannot be queried.
void* scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p != nullptr) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr)
            return nullptr;
        g_scratch_ptr[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}

}  // namespace

extern "C" {

msel_status msel_validate_bwd(const msel_scan_args* a, const msel_scan_grads* g,
                              const void* workspace, size_t workspace_bytes) {
    msel_status s = check_bwd(a, g);
    if (s != MSEL_OK) return s;
    const void* outs[] = {g->du, g->ddelta, g->dz, g->dA, g->dB, g->dC, g->dD, g->ddelta_bias,
                          g->dh0};
    const size_t need = msel_scan_bwd_workspace_bytes(a);
    if (workspace == nullptr || workspace_bytes < need) return MSEL_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MSEL_ERR_ALIGN;
    if (same_as_input(a, workspace) || workspace == g->dout || workspace == a->chunk_states)
        return MSEL_ERR_ALIAS;
    for (const void* o : outs)
        if (o != nullptr && o == workspace) return MSEL_ERR_ALIAS;
    return MSEL_OK;
}

msel_status msel_validate_conv_fwd(const msel_conv_args* a) {
    msel_status s = check_conv(a);
    if (s != MSEL_OK) return s;
    if (a->out == nullptr) return MSEL_ERR_NULL;
    if (!aligned(a->out, 16)) return MSEL_ERR_ALIGN;
    const bool state = a->width > 1 && a->state_out != nullptr;
    if (state && !aligned(a->state_out, elem_bytes(a->dtype))) return MSEL_ERR_ALIGN;
    if (conv_input(a, a->out) || (state && a->state_out == a->out)) return MSEL_ERR_ALIAS;
    // state_out may be state_in itself (the cache updated in place), no other input
    if (state && a->state_out != a->state_in && conv_input(a, a->state_out)) return MSEL_ERR_ALIAS;
    return MSEL_OK;
}

msel_status msel_validate_conv_bwd(const msel_conv_args* a, const msel_conv_grads* g) {
    msel_status s = check_conv(a);
    if (s != MSEL_OK) return s;
    if (g == nullptr || g->dout == nullptr || g->dx == nullptr) return MSEL_ERR_NULL;
    if (!aligned(g->dout, 16) || !aligned(g->dx, 16)) return MSEL_ERR_ALIGN;
    float* dstate = a->width > 1 ? g->dstate_in : nullptr;
    const void* f32[] = {g->dweight, g->dbias, dstate};
    for (const void* p : f32)
        if (p != nullptr && !aligned(p, 4)) return MSEL_ERR_ALIGN;
    const void* outs[] = {g->dx, g->dweight, g->dbias, dstate};
    for (int i = 0; i < 4; ++i) {
        const void* o = outs[i];
        if (o == nullptr) continue;
        if (conv_input(a, o) || o == g->dout) return MSEL_ERR_ALIAS;
        for (int j = 0; j < i; ++j)
            if (outs[j] == o) return MSEL_ERR_ALIAS;
    }
    return MSEL_OK;
}

msel_status msel_conv1d_fwd(const msel_conv_args* a, hipStream_t stream) {
    msel_status s = msel_validate_conv_fwd(a);
    if (s != MSEL_OK) return s;
    msel::ConvParams p = to_conv_params(a);
    p.out = a->out;
    p.state_out = a->width > 1 ? a->state_out : nullptr;
    return hip_status(msel::launch_conv_fwd(p, a->dtype == MSEL_BF16, stream));
}

msel_status msel_conv1d_bwd(const msel_conv_args* a, const msel_conv_grads* g,
                            hipStream_t stream) {
    msel_status s = msel_validate_conv_bwd(a, g);
    if (s != MSEL_OK) return s;
    msel::ConvParams p = to_conv_params(a);
    p.dout = g->dout;
    p.dx = g->dx;
    p.dw = g->dweight;
    p.dbias = g->dbias;
    p.dstate = a->width > 1 ? g->dstate_in : nullptr;
    const msel::FillList fill = {{g->dweight, g->dbias, nullptr, nullptr, nullptr, nullptr},
                                 {static_cast<size_t>(a->dim) * a->width,
                                  static_cast<size_t>(a->dim), 0, 0, 0, 0}};
    if (msel::launch_fill_zero(fill, stream) != hipSuccess) return MSEL_ERR_HIP;
    return hip_status(msel::launch_conv_bwd(p, a->dtype == MSEL_BF16, stream));
}

msel_status msel_validate_trap_bwd(const msel_scan_args* a, const msel_trap_args* tr,
                                   const msel_scan_grads* g, const msel_trap_grads* tg,
                                   const void* workspace, size_t workspace_bytes) {
    msel_status s = msel_validate_bwd(a, g, workspace, workspace_bytes);
    if (s != MSEL_OK) return s;
    if (tr == nullptr || tr->lambda == nullptr || tg == nullptr || tg->dlambda == nullptr)
        return MSEL_ERR_NULL;
    const size_t e = a->dtype == MSEL_BF16 ? 2 : 4;
    if (!aligned(tr->lambda, 16) || !aligned(tg->dlambda, 16) ||
        (tr->u_prev != nullptr && !aligned(tr->u_prev, e)) ||
        (tr->B_prev != nullptr && !aligned(tr->B_prev, e)) ||
        (tg->du_prev != nullptr && !aligned(tg->du_prev, 4)) ||
        (tg->dB_prev != nullptr && !aligned(tg->dB_prev, 4)))
        return MSEL_ERR_ALIGN;
    // every output distinct from every input, the workspace and each other
    const void* ins[] = {a->u, a->delta, a->B, a->C, a->z, a->A, a->D, a->delta_bias, a->h0,
                         a->chunk_states, g->dout, tr->lambda, tr->u_prev, tr->B_prev,
                         workspace};
    const void* outs[] = {g->du, g->ddelta, g->dz, g->dA, g->dB, g->dC, g->dD, g->ddelta_bias,
                          g->dh0, tg->dlambda, tg->du_prev, tg->dB_prev};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        if (outs[i] == nullptr) continue;
        for (const void* in : ins)
            if (in != nullptr && in == outs[i]) return MSEL_ERR_ALIAS;
        for (size_t j = 0; j < i; ++j)
            if (outs[j] == outs[i]) return MSEL_ERR_ALIAS;
    }
    return MSEL_OK;
}

msel_status msel_scan_fwd(const msel_scan_args* a, hipStream_t stream) {
    msel_status s = msel_validate_fwd(a);
    if (s != MSEL_OK) return s;
    return hip_status(msel::launch_scan_fwd(to_params(a), a->dtype == MSEL_BF16, stream));
}

msel_status msel_scan_trap_fwd(const msel_scan_args* a, const msel_trap_args* tr,
                               hipStream_t stream) {
    msel_status s = msel_validate_trap_fwd(a, tr);
    if (s != MSEL_OK) return s;
    msel::ScanParams p = to_params(a);
    p.lam = tr->lambda;
    p.u_prev = tr->u_prev;
    p.B_prev = tr->B_prev;
    return hip_status(msel::launch_scan_fwd(p, a->dtype == MSEL_BF16, stream));
}

msel_status msel_validate_complex_bwd(const msel_scan_args* a, const msel_scan_grads* g,
                                      const void* workspace, size_t workspace_bytes) {
    msel_status s = msel_validate_bwd(a, g, workspace, workspace_bytes);
    if (s != MSEL_OK) return s;
    if (a->dstate % 2 != 0) return MSEL_ERR_SHAPE;
    return MSEL_OK;
}

msel_status msel_scan_complex_bwd(const msel_scan_args* a, const msel_scan_grads* g,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
    msel_status s = msel_validate_complex_bwd(a, g, workspace, workspace_bytes);
    if (s != MSEL_OK) return s;
    const size_t DN = static_cast<size_t>(a->dim) * a->dstate;
    const size_t BNL = static_cast<size_t>(a->batch) * a->dstate * a->seqlen;
    const msel::FillList fill = {{g->dA, g->dB, g->dC, g->dD, g->ddelta_bias, nullptr},
                                 {DN, BNL, BNL, static_cast<size_t>(a->dim),
                                  static_cast<size_t>(a->dim), 0}};
    msel::GradParams gp;
    gp.dout = g->dout;
    gp.du = g->du;
    gp.ddelta = g->ddelta;
    gp.dz = g->dz;
    gp.dA = g->dA;
    gp.dB = g->dB;
    gp.dC = g->dC;
    gp.dD = g->dD;
    gp.dbias = g->ddelta_bias;
    gp.dh0 = g->dh0;
    const bool bf16 = a->dtype == MSEL_BF16;
    const msel::ScanParams p = to_params(a);
    const float* states = a->chunk_states;
    if (states == nullptr) {
        // the complex forward's chunk states, rebuilt by its chunk-carry pass into the front
        // of the workspace; the rest is laid out as with the states given
        float* H = static_cast<float*>(workspace);
        msel::ScanParams pc = p;
        pc.chunk_states = H;
        pc.final_state = nullptr;
        if (msel::launch_chunk_carry(pc, bf16, true, stream) != hipSuccess) return MSEL_ERR_HIP;
        states = H;
        workspace = static_cast<char*>(workspace) + states_bytes_aligned(a);
    }
    return hip_status(msel::launch_scan_cplx_bwd(p, gp, states, workspace, bf16, fill, stream));
}

msel_status msel_scan_complex_fwd(const msel_scan_args* a, hipStream_t stream) {
    msel_status s = msel_validate_complex_fwd(a);
    if (s != MSEL_OK) return s;
    return hip_status(msel::launch_scan_cplx_fwd(to_params(a), a->dtype == MSEL_BF16, stream));
}

msel_status msel_scan_chunk_carry(const msel_scan_args* a, hipStream_t stream) {
    msel_status s = msel_validate_chunk_carry(a);
    if (s != MSEL_OK) return s;
    return hip_status(
        msel::launch_chunk_carry(to_params(a), a->dtype == MSEL_BF16, false, stream));
}

msel_status msel_validate_trap_chunk_carry(const msel_scan_args* a, const msel_trap_args* tr) {
    msel_status s = msel_validate_chunk_carry(a);
    if (s != MSEL_OK) return s;
    if (tr == nullptr || tr->lambda == nullptr) return MSEL_ERR_NULL;
    if (!aligned(tr->lambda, 16)) return MSEL_ERR_ALIGN;
    const size_t e = a->dtype == MSEL_BF16 ? 2 : 4;
    if ((tr->u_prev != nullptr && !aligned(tr->u_prev, e)) ||
        (tr->B_prev != nullptr && !aligned(tr->B_prev, e)))
        return MSEL_ERR_ALIGN;
    const void* outs[] = {a->final_state, a->chunk_states};
    for (const void* o : outs)
        if (o != nullptr && (o == tr->lambda || o == tr->u_prev || o == tr->B_prev))
            return MSEL_ERR_ALIAS;
    return MSEL_OK;
}

msel_status msel_scan_trap_chunk_carry(const msel_scan_args* a, const msel_trap_args* tr,
                                       hipStream_t stream) {
    msel_status s = msel_validate_trap_chunk_carry(a, tr);
    if (s != MSEL_OK) return s;
    msel::ScanParams p = to_params(a);
    p.lam = tr->lambda;
    p.u_prev = tr->u_prev;
    p.B_prev = tr->B_prev;
    return hip_status(msel::launch_chunk_carry(p, a->dtype == MSEL_BF16, false, stream));
}

msel_status msel_validate_complex_chunk_carry(const msel_scan_args* a) {
    msel_status s = msel_validate_chunk_carry(a);
    if (s != MSEL_OK) return s;
    if (a->dstate % 2 != 0) return MSEL_ERR_SHAPE;  // states come in (Re, Im) pairs
    return MSEL_OK;
}

msel_status msel_scan_complex_chunk_carry(const msel_scan_args* a, hipStream_t stream) {
    msel_status s = msel_validate_complex_chunk_carry(a);
    if (s != MSEL_OK) return s;
    return hip_status(
        msel::launch_chunk_carry(to_params(a), a->dtype == MSEL_BF16, true, stream));
}

msel_status msel_scan_bwd_profiled(const msel_scan_args* a, const msel_scan_grads* g,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream,
                                   hipEvent_t ev_begin, hipEvent_t ev_end) {
    msel_status s = msel_validate_bwd(a, g, workspace, workspace_bytes);
    if (s != MSEL_OK) return s;
    return run_bwd(a, g, nullptr, nullptr, workspace, workspace_bytes, stream, ev_begin, ev_end);
}

msel_status msel_scan_trap_bwd(const msel_scan_args* a, const msel_trap_args* tr,
                               const msel_scan_grads* g, const msel_trap_grads* tg,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    msel_status s = msel_validate_trap_bwd(a, tr, g, tg, workspace, workspace_bytes);
    if (s != MSEL_OK) return s;
    return run_bwd(a, g, tr, tg, workspace, workspace_bytes, stream, nullptr, nullptr);
}

msel_status msel_ring_timeouts(unsigned long long* count) {
    if (count == nullptr) return MSEL_ERR_NULL;
    *count = 0;
    if (hipDeviceSynchronize() != hipSuccess) return MSEL_ERR_HIP;
    unsigned long long a = 0, b = 0;
    if (msel::take_ring_timeouts_bwd(&a) != hipSuccess) return MSEL_ERR_HIP;
    if (msel::take_ring_timeouts_cplx(&b) != hipSuccess) return MSEL_ERR_HIP;
    *count = a + b;
    return MSEL_OK;
}

void msel_set_ring_spin_limit(uint32_t polls) { msel::set_ring_spin_limit(polls); }

void msel_set_bwd_fused(int32_t mode) { msel::set_bwd_fused_mode(mode); }

int32_t msel_scan_bwd_fused(const msel_scan_args* a) {
    if (check_common(a) != MSEL_OK) return 0;
    return msel::bwd_plan(a->batch, a->dim, a->dstate, a->seqlen, a->chunk_states == nullptr,
                          SIZE_MAX)
                   .fused
               ? 1
               : 0;
}

int msel_checked_build(void) {
#ifdef MSEL_CHECKED
    return 1;
#else
    return 0;
#endif
}

msel_status msel_bound_violations(unsigned long long* count, uint32_t* file, uint32_t* line) {
    if (count == nullptr || file == nullptr || line == nullptr) return MSEL_ERR_NULL;
    *count = 0;
    *file = 0;
    *line = 0;
    if (hipDeviceSynchronize() != hipSuccess) return MSEL_ERR_HIP;
    using Taker = hipError_t (*)(msel::BoundsRecord*);
    // in the order of the file numbers of msel.h
    const Taker takers[] = {msel::take_bounds_fwd,  msel::take_bounds_chunk_carry,
                            msel::take_bounds_bwd,  msel::take_bounds_conv,
                            msel::take_bounds_cplx, msel::take_bounds_cplx_bwd};
    msel_status s = MSEL_OK;
    for (uint32_t i = 0; i < sizeof(takers) / sizeof(takers[0]); ++i) {
        msel::BoundsRecord r{};
        if (takers[i](&r) != hipSuccess) {
            s = MSEL_ERR_HIP;  // the other records are still read and cleared
            continue;
        }
        if (r.count != 0 && *count == 0) {
            *file = i + 1;
            *line = r.line;
        }
        *count += r.count;
    }
    return s;
}

msel_status msel_bounds_selftest(hipStream_t stream) {
    if (!msel_checked_build()) return MSEL_ERR_UNSUPPORTED;
    return msel::launch_bounds_selftest(1, stream) == hipSuccess ? MSEL_OK : MSEL_ERR_HIP;
}

msel_status msel_scan_bwd_noalloc(const msel_scan_args* a, const msel_scan_grads* g,
                                  hipStream_t stream) {
    msel_status s = check_bwd(a, g);
    if (s != MSEL_OK) return s;
    // the plan that fits in the scratch (the fused pass only if its partial sums do)
    if (msel::bwd_workspace_bytes(a->batch, a->dim, a->dstate, a->seqlen,
                                  a->chunk_states == nullptr, kScratchBytes) > kScratchBytes)
        return MSEL_ERR_TOO_LARGE;
    void* ws = scratch_on_current_device();
    if (ws == nullptr) return MSEL_ERR_HIP;
    return run_bwd(a, g, nullptr, nullptr, ws, kScratchBytes, stream, nullptr, nullptr);
}

msel_status msel_scan_bwd(const msel_scan_args* a, const msel_scan_grads* g, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    return msel_scan_bwd_profiled(a, g, workspace, workspace_bytes, stream, nullptr, nullptr);
}

}  // extern "C"
