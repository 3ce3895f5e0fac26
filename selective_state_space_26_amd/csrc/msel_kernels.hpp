// msel_kernels.hpp -- internal interface between the C ABI (msel_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msel {

// Chunk length of the scan: 64 lanes x 8 time steps.  chunk_states hold the state before
// every multiple of it; the backward and the chunk-carry pass work one chunk per wave step.
constexpr int kChunk = 512;

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
};

// All launchers enqueue on `stream` and return the hipGetLastError() after the launch.
hipError_t launch_scan_fwd(const ScanParams& p, bool bf16, hipStream_t stream);
hipError_t launch_chunk_carry(const ScanParams& p, bool bf16, hipStream_t stream);
// Backward: the summary/link passes write into `workspace` (bwd_workspace_bytes), then the
// chunk-parallel main kernel.  chunk_states may be NULL (rebuilt in the workspace).
size_t bwd_workspace_bytes(int B, int D, int N, int L, bool need_states);
// ev_begin / ev_end (either may be null) are recorded on `stream` right before and after the
// gradient kernel, so that a caller can time it alone.
hipError_t launch_scan_bwd(const ScanParams& p, const GradParams& g, const float* chunk_states,
                           void* workspace, bool bf16, hipStream_t stream,
                           hipEvent_t ev_begin = nullptr, hipEvent_t ev_end = nullptr);
// Zero-fill of up to kFillSlots float buffers in one launch (null slots are skipped).
constexpr int kFillSlots = 5;
struct FillList {
    float* p[kFillSlots];
    size_t n[kFillSlots];
};
hipError_t launch_fill_zero(const FillList& f, hipStream_t stream);

// Short causal convolution (+ bias, + SiLU when silu != 0) over rows = batch * dim rows of
// length L; W taps.  The forward reads x, state_in and writes out, state_out; the backward
// reads x, state_in, dout and writes dx, dstate and adds into dw, dbias (zeroed by the caller).
struct ConvParams {
    int64_t rows;
    int D, L, W, silu;
    int tiles;  // set by the launcher
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
// Workgroups one launch of either kernel uses (the host rejects sizes whose grid would not fit).
int64_t conv_workgroups(int64_t rows, int L, bool bf16);
hipError_t launch_conv_fwd(const ConvParams& p, bool bf16, hipStream_t stream);
hipError_t launch_conv_bwd(const ConvParams& p, bool bf16, hipStream_t stream);

}  // namespace msel
