// msel_kernels.hpp -- internal interface between the C ABI (msel_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace msel {

// Raises kernel Fn's dynamic-LDS limit to `bytes` on the current device.  The limit is a
// per-device setting, so it is made once per device (a failed attempt is retried next call).
template <auto Fn>
hipError_t allow_dynamic_lds(int bytes) {
    constexpr int kDevices = 64;
    static std::atomic<bool> done[kDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < kDevices;
    if (cached && done[dev].load(std::memory_order_acquire)) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(Fn),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && cached) done[dev].store(true, std::memory_order_release);
    return e;
}

// Compute units of the current device (256 if the query fails), looked up once per device.
inline int device_compute_units() {
    constexpr int kDevices = 64;
    static std::atomic<int> known[kDevices] = {};
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    const bool cached = dev >= 0 && dev < kDevices;
    if (cached && (cus = known[dev].load(std::memory_order_relaxed)) > 0) return cus;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 256;
    if (cached) known[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// Chunk length of the scan: 64 lanes x 8 time steps.  chunk_states hold the state before
// every multiple of it; the backward and the chunk-carry pass work one chunk per wave step.
constexpr int kChunk = 512;
// The most states per channel (the boundary's MSEL_MAX_DSTATE).
constexpr int kMaxN = 16;

struct ScanParams {
    int B, D, N, L, nchunks;
    int softplus;
    const void* u;
    const void* delta;
    const void* Bm;
    const void* Cm;
    const void* z;
    const float* A;
    const float* Dv;
    const float* bias;
    const float* h0;
    void* out;
    float* final_state;
    float* chunk_states;
    // exponential-trapezoidal variant only (null otherwise): the mixing weight [B, D, L], and
    // the inputs of the step before the first, u [B, D] and B [B, N] (null: 0)
    const void* lam = nullptr;
    const void* u_prev = nullptr;
    const void* B_prev = nullptr;
};

struct GradParams {
    const void* dout;
    void* du;
    void* ddelta;
    void* dz;
    float* dA;
    float* dB;
    float* dC;
    float* dD;
    float* dbias;
    float* dh0;
    // exponential-trapezoidal variant: gradients w.r.t. lambda [B, D, L] and the inputs of
    // the step before the first, u_prev [B, D] and B_prev [B, N] (fp32, B_prev's summed)
    void* dlam = nullptr;
    float* du_prev = nullptr;
    float* dB_prev = nullptr;
};

// The gradient kernels' LDS ring waits (scan_bwd.hip, scan_cplx_bwd.hip) are bounded: a wait
// that has polled its flag ring_spin_limit() times (each poll after an s_sleep of ~64 clocks)
// gives up, so that a protocol slip ends the kernel instead of hanging the device, and counts
// the event in a device counter of its source file, which take_ring_timeouts_* read and clear.
constexpr unsigned kRingSpinDefault = 1u << 22;  // ~0.1 s of polls at 2.4 GHz
unsigned ring_spin_limit();
void set_ring_spin_limit(unsigned polls);  // 0: the default
hipError_t take_ring_timeouts_bwd(unsigned long long* count);
hipError_t take_ring_timeouts_cplx(unsigned long long* count);

// Out-of-range indexes met by the kernels of the checked build (MSEL_IDX in msel_device.hpp),
// one record per source file; each take_bounds_* reads its file's record and clears it (the
// release build's records are always empty).
struct BoundsRecord {
    unsigned long long count;  // indexes out of range since the last read
    unsigned int line;         // source line of the first one
    unsigned int pad;
};
hipError_t take_bounds_fwd(BoundsRecord* r);
hipError_t take_bounds_chunk_carry(BoundsRecord* r);
hipError_t take_bounds_bwd(BoundsRecord* r);
hipError_t take_bounds_conv(BoundsRecord* r);
hipError_t take_bounds_cplx(BoundsRecord* r);
hipError_t take_bounds_cplx_bwd(BoundsRecord* r);
// Checked build: one kernel that forms index i of a one-element array (out of range unless
// i == 0).  The release build returns hipErrorNotSupported and launches nothing.
hipError_t launch_bounds_selftest(int i, hipStream_t stream);

// All launchers enqueue on `stream` and return the hipGetLastError() after the launch.
hipError_t launch_scan_fwd(const ScanParams& p, bool bf16, hipStream_t stream);
// The chunk-carry pass: the plain rule, the exponential-trapezoidal rule when p.lam is set, or
// the complex-valued state when cplx (N even).
hipError_t launch_chunk_carry(const ScanParams& p, bool bf16, bool cplx, hipStream_t stream);
// The complex-valued (rotational) forward: state pairs (2j, 2j+1) are complex states; N even.
hipError_t launch_scan_cplx_fwd(const ScanParams& p, bool bf16, hipStream_t stream);
// Buffers to zero before a backward's atomics (null slots are skipped).
constexpr int kFillSlots = 6;
struct FillList {
    float* p[kFillSlots];
    size_t n[kFillSlots];
};
// Grid-stride zero-fill of every slot by the threads of a launch (thread `tid` of `threads`).
__device__ __forceinline__ void zero_fill(const FillList& f, size_t tid, size_t threads) {
    for (int s = 0; s < kFillSlots; ++s) {
        float* __restrict__ p = f.p[s];
        if (p == nullptr) continue;
        for (size_t i = tid; i < f.n[s]; i += threads) p[i] = 0.0f;
    }
}
// Blocks of 256 threads for a grid-stride fill of `f` (at most 2048; 0 when there is nothing).
inline unsigned fill_blocks(const FillList& f) {
    size_t total = 0;
    for (int s = 0; s < kFillSlots; ++s)
        if (f.p[s] != nullptr) total += f.n[s];
    const size_t b = (total + 255) / 256;
    return static_cast<unsigned>(b > 2048 ? 2048 : b);
}
// Its backward from the forward's chunk states (required); the workspace is laid out as the
// real backward's with chunk states given (bwd_workspace_bytes(..., false)).
hipError_t launch_scan_cplx_bwd(const ScanParams& p, const GradParams& g,
                                const float* chunk_states, void* workspace, bool bf16,
                                const FillList& fill, hipStream_t stream);
// Backward of the plain and trapezoidal rules.  Two plans:
//  * chunk-parallel: the summary/link passes write into the workspace, then the gradient
//    kernel runs one workgroup per (batch row, chunk, channel group) and adds its sums into
//    the outputs with fp32 atomics; chunk_states may be NULL (rebuilt in the workspace);
//  * fused (plain rule, chunk states given): the gradient kernel walks the chunks from the
//    last to the first in one workgroup per (batch row, channel group), carrying the adjoint
//    itself, and stores partial sums that a reduce kernel adds in a fixed order (no summary,
//    no link, no atomics: deterministic).  Taken when the workspace holds its partial sums
//    and, by default, for at most kFusedMaxChunks chunks and enough channel groups.
constexpr int kFusedWorkgroups = 256;  // the fused grid's target (a pure function of the sizes)
constexpr int kFusedMaxChunks = 4;
struct BwdPlan {
    bool fused;
    int cgroups, per_wave;  // the fused grid
    size_t bytes;           // workspace
};
// The plan for these sizes when `cap` workspace bytes are available (need_states: the chunk
// states are rebuilt).  A pure function of its arguments and of the fused-pass setting.
BwdPlan bwd_plan(int B, int D, int N, int L, bool need_states, size_t cap);
size_t bwd_workspace_bytes(int B, int D, int N, int L, bool need_states,
                           size_t cap = SIZE_MAX);
// Fused-pass setting for later calls: 0 by size (the default), 1 wherever it applies, -1 never.
void set_bwd_fused_mode(int mode);
int bwd_fused_mode();
// ev_begin / ev_end (either may be null) are recorded on `stream` right before and after the
// gradient kernel, so that a caller can time it alone.
// `fill`: the reduction targets the chunk-parallel gradient kernel adds into, zeroed by the
// link launch.  `workspace_bytes`: the workspace's size (it decides the plan).
hipError_t launch_scan_bwd(const ScanParams& p, const GradParams& g, const float* chunk_states,
                           void* workspace, size_t workspace_bytes, bool bf16,
                           const FillList& fill, hipStream_t stream,
                           hipEvent_t ev_begin = nullptr, hipEvent_t ev_end = nullptr);
// Zero-fill of up to kFillSlots float buffers in one launch (null slots are skipped).
hipError_t launch_fill_zero(const FillList& f, hipStream_t stream);

// Division of a 31-bit unsigned value by a fixed divisor d >= 1 with one multiply-high, an add
// and a shift (the round-up method of Granlund and Montgomery): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(m, n) + n) >> l for every n < 2^31 (the sum
// then stays below 2^32).
struct FastDiv {
    uint32_t d, m, l;
};
inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return FastDiv{d, static_cast<uint32_t>(m), l};
}

// Short causal convolution (+ bias, + SiLU when silu != 0) over rows = batch * dim rows of
// length L; W taps.  The forward reads x, state_in and writes out, state_out; the backward
// reads x, state_in, dout and writes dx, dstate and adds into dw, dbias (zeroed by the caller).
struct ConvParams {
    int64_t rows;
    int D, L, W, silu;
    // set by the launcher: tiles per row, tiles per wavefront (a segment), segments per row
    int tiles, seg_tiles, segs;
    FastDiv segs_div;    // by segs
    FastDiv dim_div;     // by D
    const void* x;
    const float* w;
    const float* bias;
    const void* state_in;
    void* out;
    void* state_out;
    const void* dout;
    void* dx;
    float* dw;
    float* dbias;
    float* dstate;
};
// Wavefronts one launch of either kernel uses; the host rejects sizes above kMaxConvWaves
// wavefronts (their indices must stay below 2^31).
constexpr int64_t kMaxConvWaves = (int64_t(1) << 31) - 1;
int64_t conv_waves(int64_t rows, int L, bool bf16);
hipError_t launch_conv_fwd(const ConvParams& p, bool bf16, hipStream_t stream);
hipError_t launch_conv_bwd(const ConvParams& p, bool bf16, hipStream_t stream);

}  // namespace msel
