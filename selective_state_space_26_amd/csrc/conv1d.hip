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
// Work split: tiles of 64*K consecutive steps of one (b, d) row, K = two 16-byte vectors per
// lane (16 bf16 or 8 fp32 values); lane l holds steps [t0 + l*K, t0 + (l+1)*K).  The forward
// runs one wavefront per tile.  The backward runs one wavefront per segment of consecutive
// tiles of a row, with the next tile's loads in flight while one is computed, and adds its
// tap and bias sums with one atomic per segment.  The W-1 inputs before a lane's first step
// come from lane l-1 through a wave-wide DPP shift; lane 0 takes them from the previous tile
// (a wave-uniform load at a segment's start, registers inside it) or from state_in for the
// row's first tile.  The backward also needs dpre at the W-1 steps after a lane's last one:
// lane l+1 provides them, and lane 63 recomputes them from lane 0 of the next tile.  The first
// tile's wavefront is the only reader of state_in and the only writer of state_out, after its
// reads, so the cache may be updated in place.  Accesses are plain cached ones: the
// non-temporal hint measured slower for these streams.
// seqlen 1 (the decode step) runs a separate kernel with one thread per row.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "msel_device.hpp"
#include "msel_kernels.hpp"

namespace msel {

namespace {

constexpr int kConvWaves = 4;  // wavefronts per workgroup
// wavefronts a launch aims for: 16 per CU of the 256 (at most 32 fit)
constexpr int64_t kConvTargetWaves = 4096;

template <typename T>
constexpr int conv_k() { return 2 * Elem<T>::kPerVec; }

// d/dp of p * sigmoid(p)
__device__ __forceinline__ float dsilu(float p) {
    const float s = sigmoid_f(p);
    return s * fmaf(p, 1.0f - s, 1.0f);
}

__device__ __forceinline__ uint32_t div_by(uint32_t n, const FastDiv& f) {
    return (__umulhi(n, f.m) + n) >> f.l;
}

// A wavefront's work: tiles [tile0, tile0 + ntiles) of one (b, d) row.
struct Seg {
    int64_t row;  // b * dim + d
    int d;
    int seg;      // index of the segment in its row
    int tile0;
    int ntiles;
};

__device__ __forceinline__ bool seg_of(const ConvParams& p, Seg& s) {
    const uint32_t wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t wave = blockIdx.x * kConvWaves + wid;  // < 2^31: checked on the host
    if (wave >= static_cast<uint32_t>(p.rows) * static_cast<uint32_t>(p.segs)) return false;
    const uint32_t row = div_by(wave, p.segs_div);
    s.row = MSEL_IDX(static_cast<int64_t>(row), p.rows);
    s.seg = static_cast<int>(wave - row * static_cast<uint32_t>(p.segs));
    s.d = MSEL_IDX(static_cast<int>(row - div_by(row, p.dim_div) * static_cast<uint32_t>(p.D)),
                   p.D);
    s.tile0 = s.seg * p.seg_tiles;
    s.ntiles = min(p.seg_tiles, p.tiles - s.tile0);
    return true;
}

// Input at step t of the extended sequence [state_in, x]: t < 0 reads the state (entry
// t + H), or 0 without one.  Wave-uniform t.
template <typename T, int H>
__device__ __forceinline__ float input_at(const T* __restrict__ xr, const T* st, int t) {
    if (t >= 0) return Elem<T>::load1(xr + t);
    return st != nullptr ? Elem<T>::load1(st + H + (MSEL_IDX(H + t, H) - H)) : 0.0f;
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
    Seg sg;  // the forward's segments are single tiles
    if (!seg_of(p, sg)) return;
    const int L = p.L;
    const int lane = lane_id();
    const int tw = sg.tile0 * 64 * K;
    const int t0 = tw + lane * K;
    const T* __restrict__ xr = static_cast<const T*>(p.x) + sg.row * L;
    const T* st = (H > 0 && p.state_in != nullptr)
                      ? static_cast<const T*>(p.state_in) + sg.row * H : nullptr;

    float v[K];
    load_k_cached<T, K, VEC>(xr, t0, L, v);
    float wk[W];
#pragma unroll
    for (int i = 0; i < W; ++i)
        wk[i] = p.w[MSEL_IDX(static_cast<size_t>(sg.d) * W + i, static_cast<size_t>(p.D) * W)];
    const float b = p.bias != nullptr ? p.bias[sg.d] : 0.0f;

    // the H inputs before each lane's first step, oldest first
    float prev[HA];
#pragma unroll
    for (int j = 0; j < H; ++j) prev[j] = shift_up(v[K - H + j], input_at<T, H>(xr, st, tw - H + j));

    float o[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float pre = pre_at<W, K>(wk, b, prev, v, k);
        o[k] = SILU ? pre * sigmoid_f(pre) : pre;
    }
    store_k<T, K, VEC, false>(static_cast<T*>(p.out) + sg.row * L, t0, L, o);

    // the cache after the call: the last H entries of [state_in, x]
    if (H > 0 && sg.seg == 0 && p.state_out != nullptr && lane < H) {
        const int t = L - H + lane;
        float s = 0.0f;
        if (t >= 0)
            s = Elem<T>::load1(xr + MSEL_IDX(t, L));
        else if (st != nullptr)
            s = Elem<T>::load1(st + H + (MSEL_IDX(H + t, H) - H));
        Elem<T>::store1(static_cast<T*>(p.state_out) + sg.row * H + MSEL_IDX(lane, H), s);
    }
}

template <typename T, int W, bool SILU, bool VEC>
__global__ __launch_bounds__(64 * kConvWaves) void conv_bwd_kernel(ConvParams p) {
    constexpr int K = conv_k<T>();
    constexpr int H = W - 1;
    constexpr int HA = H > 0 ? H : 1;
    constexpr int TILE = 64 * K;
    Seg sg;
    if (!seg_of(p, sg)) return;
    const int L = p.L;
    const int lane = lane_id();
    const T* __restrict__ xr = static_cast<const T*>(p.x) + sg.row * L;
    const T* __restrict__ gr = static_cast<const T*>(p.dout) + sg.row * L;
    T* __restrict__ dxr = static_cast<T*>(p.dx) + sg.row * L;
    const T* st = (H > 0 && p.state_in != nullptr)
                      ? static_cast<const T*>(p.state_in) + sg.row * H : nullptr;
    int t0 = sg.tile0 * TILE + lane * K;

    Raw<T, K> cx, cg, nx, ng;
    load_raw<T, K, VEC>(xr, t0, L, cx);
    load_raw<T, K, VEC>(gr, t0, L, cg);
    float wk[W];
#pragma unroll
    for (int i = 0; i < W; ++i)
        wk[i] = p.w[MSEL_IDX(static_cast<size_t>(sg.d) * W + i, static_cast<size_t>(p.D) * W)];
    const float b = p.bias != nullptr ? p.bias[sg.d] : 0.0f;
    float halo[HA];
#pragma unroll
    for (int j = 0; j < H; ++j) halo[j] = input_at<T, H>(xr, st, sg.tile0 * TILE - H + j);
    // sums over the segment: lane partials of dw[i] and of dbias (index W)
    float part[W + 1];
#pragma unroll
    for (int i = 0; i <= W; ++i) part[i] = 0.0f;

    for (int i = 0; i < sg.ntiles; ++i, t0 += TILE) {
        // the next tile in flight while this one is computed (zeros past the row's end); its
        // first steps also complete this tile's last dpre values
        load_raw<T, K, VEC>(xr, t0 + TILE, L, nx);
        load_raw<T, K, VEC>(gr, t0 + TILE, L, ng);
        float v[K], g[K];
        unpack<T, K>(cx, v);
        unpack<T, K>(cg, g);
        float prev[HA];
#pragma unroll
        for (int j = 0; j < H; ++j) prev[j] = shift_up(v[K - H + j], halo[j]);

        // dpre at the lane's own steps (0 past the end: dout reads 0 there)
        float dp[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float pre = pre_at<W, K>(wk, b, prev, v, k);
            dp[k] = SILU ? g[k] * dsilu(pre) : g[k];
        }

        // dpre at the H steps after the tile, for lane 63, from the window [x of lane 63's
        // last H steps, x of the next tile's first H steps (lane 0 of the next tile)]
        float nxt[HA];
        if constexpr (H > 0) {
            float ext[2 * H], gn[H];
            {
                float vn[K], gnk[K];
                unpack<T, K>(nx, vn);
                unpack<T, K>(ng, gnk);
#pragma unroll
                for (int j = 0; j < H; ++j) {
                    ext[H + j] = readlane(vn[j], 0);
                    gn[j] = readlane(gnk[j], 0);
                }
            }
#pragma unroll
            for (int j = 0; j < H; ++j) ext[j] = readlane(v[K - H + j], 63);
#pragma unroll
            for (int j = 0; j < H; ++j) {
                float pre = b;
#pragma unroll
                for (int q = 0; q < W; ++q) pre = fmaf(wk[q], ext[j + q], pre);
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
            for (int q = 0; q < W; ++q) {
                const int e = k + H - q;
                acc = fmaf(wk[q], e < K ? dp[e] : nxt[e - K], acc);
            }
            dx[k] = acc;
        }
        store_k<T, K, VEC, false>(dxr, t0, L, dx);

        // gradient w.r.t. the incoming state: entry j (step j - H) meets tap j - m at step
        // m <= j, all inside lane 0 of the row's first tile
        if (H > 0 && sg.tile0 + i == 0 && p.dstate != nullptr) {
            float d0[HA];
#pragma unroll
            for (int m = 0; m < H; ++m) d0[m] = readlane(dp[m], 0);
            if (lane == 0) {
#pragma unroll
                for (int j = 0; j < H; ++j) {
                    float acc = 0.0f;
#pragma unroll
                    for (int m = 0; m <= j; ++m) acc = fmaf(wk[j - m], d0[m], acc);
                    p.dstate[sg.row * H + MSEL_IDX(j, H)] = acc;
                }
            }
        }

        // dw[q] gathers dpre * xe[step + q], dbias gathers dpre
#pragma unroll
        for (int k = 0; k < K; ++k) {
#pragma unroll
            for (int q = 0; q < W; ++q) {
                const int e = k + q;
                part[q] = fmaf(dp[k], e < H ? prev[e] : v[e - H], part[q]);
            }
            part[W] += dp[k];
        }
#pragma unroll
        for (int j = 0; j < H; ++j) halo[j] = readlane(v[K - H + j], 63);
        cx = nx;
        cg = ng;
    }

    if (p.dw != nullptr || p.dbias != nullptr) {
        float tot[W + 1];
#pragma unroll
        for (int q = 0; q <= W; ++q) tot[q] = wave_sum_fused(part[q]);
        // one vector atomic per segment: lane q < W adds dw[d, q], lane 63 adds dbias[d]
        float* dst = nullptr;
        float val = 0.0f;
#pragma unroll
        for (int q = 0; q < W; ++q)
            if (lane == q && p.dw != nullptr) {
                dst = p.dw + MSEL_IDX(static_cast<size_t>(sg.d) * W + q, static_cast<size_t>(p.D) * W);
                val = tot[q];
            }
        if (lane == 63 && p.dbias != nullptr) {
            dst = p.dbias + sg.d;
            val = tot[W];
        }
        if (dst != nullptr) unsafeAtomicAdd(dst, val);
    }
}

// The recurrent (decode) step, seqlen 1: one thread per (b, d) row.  It reads the row's
// state and input, writes the output and the shifted state [state[1..H), x] -- after its own
// reads, so the state may be updated in place.
template <typename T, int W, bool SILU>
__global__ __launch_bounds__(256) void conv_step_kernel(ConvParams p) {
    constexpr int H = W - 1;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (row >= p.rows) return;
    const int d = MSEL_IDX(static_cast<int>(row % p.D), p.D);
    const T* st = (H > 0 && p.state_in != nullptr)
                      ? static_cast<const T*>(p.state_in) + row * H : nullptr;
    float win[W];  // [state, x]
#pragma unroll
    for (int j = 0; j < H; ++j) win[j] = st != nullptr ? Elem<T>::load1(st + j) : 0.0f;
    win[H] = Elem<T>::load1(static_cast<const T*>(p.x) + row);
    float pre = p.bias != nullptr ? p.bias[d] : 0.0f;
#pragma unroll
    for (int i = 0; i < W; ++i)
        pre = fmaf(p.w[MSEL_IDX(static_cast<size_t>(d) * W + i, static_cast<size_t>(p.D) * W)],
                   win[i], pre);
    Elem<T>::store1(static_cast<T*>(p.out) + row, SILU ? pre * sigmoid_f(pre) : pre);
    if (H > 0 && p.state_out != nullptr) {
        T* so = static_cast<T*>(p.state_out) + row * H;
#pragma unroll
        for (int j = 0; j < H; ++j) Elem<T>::store1(so + j, win[j + 1]);
    }
}

template <typename T, int W, bool SILU>
hipError_t conv_go(const ConvParams& p, bool bwd, hipStream_t stream) {
    const bool vec = p.L % Elem<T>::kPerVec == 0;
    const int64_t waves = p.rows * p.segs;
    const dim3 grid(static_cast<unsigned>((waves + kConvWaves - 1) / kConvWaves));
    const dim3 block(64 * kConvWaves);
    if (!bwd && p.L == 1) {
        hipLaunchKernelGGL((conv_step_kernel<T, W, SILU>),
                           dim3(static_cast<unsigned>((p.rows + 255) / 256)), dim3(256), 0, stream,
                           p);
        return hipGetLastError();
    }
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
    // tiles per wavefront.  The forward takes one: wavefronts that run together then stream
    // one contiguous stretch of memory, which measured faster than many row-wise streams.  The
    // backward walks segments of several tiles with the next one in flight, so that it adds
    // its tap/bias sums once per segment: the tiles of one channel run at the same time, and
    // one atomic per tile on the same few addresses measured as a large share of its time.
    const int64_t total = p.rows * p.tiles;
    p.seg_tiles = bwd ? static_cast<int>(std::min<int64_t>(
                            p.tiles, std::max<int64_t>(1, (total + kConvTargetWaves - 1) /
                                                              kConvTargetWaves)))
                      : 1;
    p.segs = (p.tiles + p.seg_tiles - 1) / p.seg_tiles;
    if (p.rows * p.segs > kMaxConvWaves) return hipErrorInvalidValue;
    p.segs_div = make_fastdiv(static_cast<uint32_t>(p.segs));
    p.dim_div = make_fastdiv(static_cast<uint32_t>(p.D));
    return p.silu ? conv_width<T, true>(p, bwd, stream) : conv_width<T, false>(p, bwd, stream);
}

}  // namespace

int64_t conv_waves(int64_t rows, int L, bool bf16) {
    // the most a launch uses: one wavefront per tile
    const int64_t per_tile = 64 * (bf16 ? conv_k<bf16_t>() : conv_k<float>());
    return rows * ((L + per_tile - 1) / per_tile);
}

hipError_t launch_conv_fwd(const ConvParams& p, bool bf16, hipStream_t stream) {
    return bf16 ? conv_dispatch<bf16_t>(p, false, stream) : conv_dispatch<float>(p, false, stream);
}

hipError_t launch_conv_bwd(const ConvParams& p, bool bf16, hipStream_t stream) {
    return bf16 ? conv_dispatch<bf16_t>(p, true, stream) : conv_dispatch<float>(p, true, stream);
}

MSEL_BOUNDS_TAKER(take_bounds_conv)

}  // namespace msel
