// conv1d.hip -- the short causal depthwise convolution + bias + SiLU that produces the scan's
// input, forward and backward (the backward recomputes the pre-activation from x).
//
// The selective SSM block applies an input projection, a short convolution, an activation,
// the scan and an output projection, and recomputes the convolution and activation outputs in
// the backward instead of storing them (page 4, Gu & Dao "Mamba", Appendix D, Memory
// paragraph).  The layer's cache keeps the convolutional state next to the SSM state (page 1,
// "A Secret Weapon For mamba paper", cache paragraph).
//
// Both kernels stream HBM.  Per element the forward reads x and writes out; the backward reads
// x and dout and writes dx.  W multiply-adds and one exp per element are far below the chip's
// ALU rate, so the design goal is full-width coalesced 16-byte accesses and enough bytes in
// flight, nothing else.
//
// Work split: one wavefront per tile of 64*K consecutive steps of one (b, d) row, K = two
// 16-byte vectors per lane (16 bf16 or 8 fp32 values).  Lane l holds steps
// [t0 + l*K, t0 + (l+1)*K).  The W-1 inputs before a lane's first step come from lane l-1
// through a wave-wide DPP shift; lane 0 takes them from a wave-uniform load of the previous
// tile's last inputs, or of state_in for the first tile.  The backward also needs dpre at the
// W-1 steps after a lane's last one: lane l+1 provides them, and lane 63 recomputes them from
// the next tile's first inputs.  The first tile's wavefront is the only reader of state_in
// and the only writer of state_out, after its reads, so the cache may be updated in place.
#include <hip/hip_runtime.h>

#include "msel_device.hpp"
#include "msel_kernels.hpp"

namespace msel {

namespace {

constexpr int kConvWaves = 4;  // wavefronts per workgroup

template <typename T>
constexpr int conv_k() { return 2 * Elem<T>::kPerVec; }

// d/dp of p * sigmoid(p)
__device__ __forceinline__ float dsilu(float p) {
    const float s = sigmoid_f(p);
    return s * fmaf(p, 1.0f - s, 1.0f);
}

struct Tile {
    int64_t row;  // b * dim + d
    int d;
    int tile;     // index of the tile in its row
    int tw;       // first step of the tile
    int t0;       // first step of this lane
};

template <typename T>
__device__ __forceinline__ bool tile_of(const ConvParams& p, Tile& w) {
    constexpr int K = conv_k<T>();
    const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * kConvWaves + wid;
    if (wave >= p.rows * p.tiles) return false;
    w.row = wave / p.tiles;
    w.tile = static_cast<int>(wave - w.row * p.tiles);
    w.d = static_cast<int>(w.row % p.D);
    w.tw = w.tile * 64 * K;
    w.t0 = w.tw + lane_id() * K;
    return true;
}

// Input at step t of the extended sequence [state_in, x]: t < 0 reads the state (entry
// t + H), or 0 without one.  Wave-uniform t.
template <typename T, int H>
__device__ __forceinline__ float input_at(const T* __restrict__ xr, const T* st, int t) {
    if (t >= 0) return Elem<T>::load1(xr + t);
    return st != nullptr ? Elem<T>::load1(st + H + t) : 0.0f;
}

// pre-activation of lane step k from the window [prev[0..H), v[0..K)]
template <int W, int K>
__device__ __forceinline__ float pre_at(const float (&w)[W], float b, const float* prev,
                                        const float (&v)[K], int k) {
    constexpr int H = W - 1;
    float acc = b;
#pragma unroll
    for (int i = 0; i < W; ++i) {
        const int e = k + i;
        acc = fmaf(w[i], e < H ? prev[e] : v[e - H], acc);
    }
    return acc;
}

template <typename T, int W, bool SILU, bool VEC>
__global__ __launch_bounds__(64 * kConvWaves) void conv_fwd_kernel(ConvParams p) {
    constexpr int K = conv_k<T>();
    constexpr int H = W - 1;
    constexpr int HA = H > 0 ? H : 1;
    Tile tl;
    if (!tile_of<T>(p, tl)) return;
    const int L = p.L;
    const T* __restrict__ xr = static_cast<const T*>(p.x) + tl.row * L;
    const T* st = (H > 0 && p.state_in != nullptr)
                      ? static_cast<const T*>(p.state_in) + tl.row * H : nullptr;

    float v[K];
    load_k<T, K, VEC>(xr, tl.t0, L, v, 0.0f);
    float wk[W];
#pragma unroll
    for (int i = 0; i < W; ++i) wk[i] = p.w[static_cast<size_t>(tl.d) * W + i];
    const float b = p.bias != nullptr ? p.bias[tl.d] : 0.0f;

    // the H inputs before each lane's first step, oldest first
    float prev[HA];
#pragma unroll
    for (int j = 0; j < H; ++j)
        prev[j] = shift_up(v[K - H + j], input_at<T, H>(xr, st, tl.tw - H + j));

    float o[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float pre = pre_at<W, K>(wk, b, prev, v, k);
        o[k] = SILU ? pre * sigmoid_f(pre) : pre;
    }
    store_k<T, K, VEC>(static_cast<T*>(p.out) + tl.row * L, tl.t0, L, o);

    // the cache after the call: the last H entries of [state_in, x]
    if (H > 0 && tl.tile == 0 && p.state_out != nullptr && lane_id() < H) {
        const int t = L - H + lane_id();
        float s = 0.0f;
        if (t >= 0)
            s = Elem<T>::load1(xr + t);
        else if (st != nullptr)
            s = Elem<T>::load1(st + H + t);
        Elem<T>::store1(static_cast<T*>(p.state_out) + tl.row * H + lane_id(), s);
    }
}

template <typename T, int W, bool SILU, bool VEC>
__global__ __launch_bounds__(64 * kConvWaves) void conv_bwd_kernel(ConvParams p) {
    constexpr int K = conv_k<T>();
    constexpr int H = W - 1;
    constexpr int HA = H > 0 ? H : 1;
    Tile tl;
    if (!tile_of<T>(p, tl)) return;
    const int L = p.L;
    const int lane = lane_id();
    const T* __restrict__ xr = static_cast<const T*>(p.x) + tl.row * L;
    const T* __restrict__ gr = static_cast<const T*>(p.dout) + tl.row * L;
    const T* st = (H > 0 && p.state_in != nullptr)
                      ? static_cast<const T*>(p.state_in) + tl.row * H : nullptr;

    float v[K], g[K];
    load_k<T, K, VEC>(xr, tl.t0, L, v, 0.0f);
    load_k<T, K, VEC>(gr, tl.t0, L, g, 0.0f);
    float wk[W];
#pragma unroll
    for (int i = 0; i < W; ++i) wk[i] = p.w[static_cast<size_t>(tl.d) * W + i];
    const float b = p.bias != nullptr ? p.bias[tl.d] : 0.0f;

    float prev[HA];
#pragma unroll
    for (int j = 0; j < H; ++j)
        prev[j] = shift_up(v[K - H + j], input_at<T, H>(xr, st, tl.tw - H + j));

    // dpre at the lane's own steps (0 past the end: dout reads 0 there)
    float dp[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float pre = pre_at<W, K>(wk, b, prev, v, k);
        dp[k] = SILU ? g[k] * dsilu(pre) : g[k];
    }

    // dpre at the H steps after the tile, for lane 63: window [x of lane 63's last H steps,
    // x of the next tile's first H steps]
    float nxt[HA];
    if constexpr (H > 0) {
        const int tn = tl.tw + 64 * K;
        float ext[2 * H], gn[H];
#pragma unroll
        for (int j = 0; j < H; ++j) {
            ext[j] = readlane(v[K - H + j], 63);
            const bool in = tn + j < L;
            ext[H + j] = in ? Elem<T>::load1(xr + tn + j) : 0.0f;
            gn[j] = in ? Elem<T>::load1(gr + tn + j) : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < H; ++j) {
            float pre = b;
#pragma unroll
            for (int i = 0; i < W; ++i) pre = fmaf(wk[i], ext[j + i], pre);
            const float dpn = SILU ? gn[j] * dsilu(pre) : gn[j];
            nxt[j] = shift_down(dp[j], dpn);
        }
    }

    // dx at step s gathers w[i] * dpre[s + H - i]
    float dx[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < W; ++i) {
            const int e = k + H - i;
            acc = fmaf(wk[i], e < K ? dp[e] : nxt[e - K], acc);
        }
        dx[k] = acc;
    }
    store_k<T, K, VEC>(static_cast<T*>(p.dx) + tl.row * L, tl.t0, L, dx);

    // gradient w.r.t. the incoming state: entry j (step j - H) meets tap j - m at step m <= j
    if (H > 0 && tl.tile == 0 && p.dstate != nullptr) {
        float d0[HA];
#pragma unroll
        for (int m = 0; m < H; ++m) d0[m] = readlane(dp[m], 0);
        if (lane == 0) {
#pragma unroll
            for (int j = 0; j < H; ++j) {
                float acc = 0.0f;
#pragma unroll
                for (int m = 0; m <= j; ++m) acc = fmaf(wk[j - m], d0[m], acc);
                p.dstate[tl.row * H + j] = acc;
            }
        }
    }

    // dw[i] = sum over steps of dpre * xe[step + i], dbias = sum of dpre
    if (p.dw != nullptr || p.dbias != nullptr) {
        float part[W + 1];
#pragma unroll
        for (int i = 0; i <= W; ++i) part[i] = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
#pragma unroll
            for (int i = 0; i < W; ++i) {
                const int e = k + i;
                part[i] = fmaf(dp[k], e < H ? prev[e] : v[e - H], part[i]);
            }
            part[W] += dp[k];
        }
        float tot[W + 1];
#pragma unroll
        for (int i = 0; i <= W; ++i) tot[i] = wave_sum_fused(part[i]);
        // one vector atomic: lane i < W adds dw[d, i], lane 63 adds dbias[d]
        float* dst = nullptr;
        float val = 0.0f;
#pragma unroll
        for (int i = 0; i < W; ++i)
            if (lane == i && p.dw != nullptr) {
                dst = p.dw + static_cast<size_t>(tl.d) * W + i;
                val = tot[i];
            }
        if (lane == 63 && p.dbias != nullptr) {
            dst = p.dbias + tl.d;
            val = tot[W];
        }
        if (dst != nullptr) unsafeAtomicAdd(dst, val);
    }
}

template <typename T, int W, bool SILU>
hipError_t conv_go(const ConvParams& p, bool bwd, hipStream_t stream) {
    const bool vec = p.L % Elem<T>::kPerVec == 0;
    const int64_t waves = p.rows * p.tiles;
    const dim3 grid(static_cast<unsigned>((waves + kConvWaves - 1) / kConvWaves));
    const dim3 block(64 * kConvWaves);
    if (bwd) {
        if (vec)
            hipLaunchKernelGGL((conv_bwd_kernel<T, W, SILU, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((conv_bwd_kernel<T, W, SILU, false>), grid, block, 0, stream, p);
    } else {
        if (vec)
            hipLaunchKernelGGL((conv_fwd_kernel<T, W, SILU, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((conv_fwd_kernel<T, W, SILU, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

template <typename T, bool SILU>
hipError_t conv_width(const ConvParams& p, bool bwd, hipStream_t stream) {
    switch (p.W) {
        case 1: return conv_go<T, 1, SILU>(p, bwd, stream);
        case 2: return conv_go<T, 2, SILU>(p, bwd, stream);
        case 3: return conv_go<T, 3, SILU>(p, bwd, stream);
        case 4: return conv_go<T, 4, SILU>(p, bwd, stream);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t conv_dispatch(ConvParams p, bool bwd, hipStream_t stream) {
    p.tiles = static_cast<int>((static_cast<int64_t>(p.L) + 64 * conv_k<T>() - 1) /
                               (64 * conv_k<T>()));
    return p.silu ? conv_width<T, true>(p, bwd, stream) : conv_width<T, false>(p, bwd, stream);
}

}  // namespace

int64_t conv_workgroups(int64_t rows, int L, bool bf16) {
    const int64_t per_tile = 64 * (bf16 ? conv_k<bf16_t>() : conv_k<float>());
    const int64_t waves = rows * ((L + per_tile - 1) / per_tile);
    return (waves + kConvWaves - 1) / kConvWaves;
}

hipError_t launch_conv_fwd(const ConvParams& p, bool bf16, hipStream_t stream) {
    return bf16 ? conv_dispatch<bf16_t>(p, false, stream) : conv_dispatch<float>(p, false, stream);
}

hipError_t launch_conv_bwd(const ConvParams& p, bool bf16, hipStream_t stream) {
    return bf16 ? conv_dispatch<bf16_t>(p, true, stream) : conv_dispatch<float>(p, true, stream);
}

}  // namespace msel
