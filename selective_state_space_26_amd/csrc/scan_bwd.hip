// scan_bwd.hip -- backward selective scan with recomputation, for gfx950.
//
// Page 1 and page 4 (Appendix D, Memory paragraph): the intermediate states are not stored
// but recomputed in the backward pass when the inputs are loaded from HBM into on-chip
// memory.  Only the chunk-boundary states H_c (one per kChunk steps, from the forward or the
// chunk-carry pass) are read; inside a chunk the states are rebuilt in registers.
//
// Gradients of a loss with respect to the inputs, given dout (a = exp(Delta A), p = Delta B u,
// y = C.h + D u before the gate, s = sigmoid(z)):
//   dy_t  = dout_t * z s                 dz_t = dout_t * y_t * s (1 + z (1 - s))
//   lam_t = C_t dy_t + a_{t+1} lam_{t+1} (adjoint of h_t, zero beyond the last step)
//   dC_t += dy_t h_t      dB_t += lam_t Delta_t u_t      (summed over channels)
//   g_t   = lam_t h_{t-1} a_t          dA += g_t Delta_t (summed over batch and time)
//   dDelta_t = sum_n (g_t A + lam_t B_t u_t)   du_t = sum_n lam_t Delta_t B_t + dy_t D
//   ddelta_t = dDelta_t * sigmoid(delta_t + bias) with the softplus, dbias += ddelta_t
//   dD += dy_t u_t       dh0 = a_0 lam_0
//
// Layout: a workgroup holds kBwdWaves wavefronts, one per channel of the same batch row, and
// walks the chunks from last to first.  Lane l covers steps [c*T + l*K, c*T + (l+1)*K).  Per
// state n: forward pass 1 + DPP scan + pass 2 rebuilds h_t from H_c; the adjoint runs the same
// way in reverse (lane-local chain, DPP suffix scan, replay) starting from the carry of the
// chunk after it.  dB and dC are summed over the workgroup's channels with LDS atomics into a
// double-buffered [K][64] tile (one buffer per state, alternating), then flushed to HBM with
// fp32 global atomics.  dA partials stay lane-private in LDS until the end.
#include "msel_device.hpp"
#include "msel_kernels.hpp"

namespace msel {

constexpr int kBwdWaves = 4;
constexpr int kMaxN = 16;

template <typename T, bool VEC, bool HAS_Z, bool SOFTPLUS>
__global__ __launch_bounds__(64 * kBwdWaves) void scan_bwd_kernel(ScanParams p, GradParams g,
                                                                   const float* __restrict__ cst) {
    constexpr int K = kChunk / 64;
    constexpr int W = kBwdWaves;
    constexpr int KP = 65;      // padded lane stride of the [K][64] accumulator tile
    constexpr int ACC = K * KP;
    __shared__ float accB[2][ACC];
    __shared__ float accC[2][ACC];
    __shared__ float accA[W][kMaxN][64];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = blockIdx.y;
    const int d_raw = blockIdx.x * W + wave;
    const bool active = d_raw < p.D;
    const int d = active ? d_raw : 0;
    const int N = p.N;
    const int L = p.L;
    const int nch = p.nchunks;

    for (int i = tid; i < 2 * ACC; i += 64 * W) {
        (&accB[0][0])[i] = 0.0f;
        (&accC[0][0])[i] = 0.0f;
    }
    for (int i = tid; i < W * kMaxN * 64; i += 64 * W) (&accA[0][0][0])[i] = 0.0f;
    __syncthreads();

    const size_t ch = static_cast<size_t>(b) * p.D + d;
    const size_t row = ch * L;
    const T* __restrict__ u = static_cast<const T*>(p.u) + row;
    const T* __restrict__ dl = static_cast<const T*>(p.delta) + row;
    const T* __restrict__ zr = HAS_Z ? static_cast<const T*>(p.z) + row : nullptr;
    const T* __restrict__ go = static_cast<const T*>(g.dout) + row;
    T* __restrict__ du_o = static_cast<T*>(g.du) + row;
    T* __restrict__ dd_o = static_cast<T*>(g.ddelta) + row;
    T* __restrict__ dz_o = HAS_Z ? static_cast<T*>(g.dz) + row : nullptr;
    const T* __restrict__ Bb = static_cast<const T*>(p.Bm) + static_cast<size_t>(b) * N * L;
    const T* __restrict__ Cb = static_cast<const T*>(p.Cm) + static_cast<size_t>(b) * N * L;
    const float bias = p.bias ? p.bias[d] : 0.0f;
    const float Dd = p.Dv ? p.Dv[d] : 0.0f;
    const float* __restrict__ Arow = p.A + static_cast<size_t>(d) * N;
    const float* __restrict__ Hrow = cst + ch * nch * N;

    float G = 0.0f;  // lane n: a_t lam_t at the first step of the chunk after the current one
    float dD_acc = 0.0f, dbias_acc = 0.0f;
    int it = 0;      // running (chunk, state) counter: selects the accumulator buffer

    for (int c = nch - 1; c >= 0; --c) {
        const int t0 = c * kChunk + lane * K;
        float dt[K], dtu[K], uu[K], dy[K], sB[K], sgA[K], dsp[K];
        float y[HAS_Z ? K : 1], gz[HAS_Z ? K : 1];
        float sum_dt = 0.0f, dt_next = 0.0f;
        if (active) {
            float dd[K], gg[K];
            load_k<T, K, VEC>(u, t0, L, uu, 0.0f);
            load_k<T, K, VEC>(dl, t0, L, dd, 0.0f);
            load_k<T, K, VEC>(go, t0, L, gg, 0.0f);
            float zz[HAS_Z ? K : 1];
            if constexpr (HAS_Z) load_k<T, K, VEC>(zr, t0, L, zz, 0.0f);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const bool valid = t0 + k < L;
                const float x = dd[k] + bias;
                const float v = SOFTPLUS ? softplus_f(x) : x;
                dt[k] = valid ? v : 0.0f;
                dsp[k] = SOFTPLUS ? sigmoid_f(x) : 1.0f;
                dtu[k] = dt[k] * uu[k];
                sum_dt += dt[k];
                if constexpr (HAS_Z) {
                    const float s = sigmoid_f(zz[k]);
                    dy[k] = gg[k] * zz[k] * s;
                    gz[k] = gg[k] * s * fmaf(zz[k], 1.0f - s, 1.0f);
                    y[k] = Dd * uu[k];
                } else {
                    dy[k] = gg[k];
                }
                dD_acc = fmaf(dy[k], uu[k], dD_acc);
                sB[k] = 0.0f;
                sgA[k] = 0.0f;
            }
            dt_next = dpp<kWaveShl1, 0xf>(0.0f, dt[0]);  // Delta at the next lane's first step
        }

        for (int n = 0; n < N; ++n, ++it) {
            const int buf = it & 1;
            if (active) {
                const float An = Arow[n];
                const float An2 = An * kLog2e;
                float bv[K], cv[K];
                load_k_cached<T, K, VEC>(Bb + static_cast<size_t>(n) * L, t0, L, bv);
                load_k_cached<T, K, VEC>(Cb + static_cast<size_t>(n) * L, t0, L, cv);
                // forward recompute of the states inside the chunk
                float a[K], bb[K], hs[K];
                float h = 0.0f;
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    a[k] = exp2_hw(dt[k] * An2);
                    bb[k] = dtu[k] * bv[k];
                    h = fmaf(a[k], h, bb[k]);
                }
                float P = exp2_hw(An2 * sum_dt);
                float S = h;
                wave_scan_fwd(P, S);
                float Pex, Sex;
                wave_shift_fwd(P, S, Pex, Sex);
                const float hin = fmaf(Pex, Hrow[static_cast<size_t>(c) * N + n], Sex);
                h = hin;
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    h = fmaf(a[k], h, bb[k]);
                    hs[k] = h;
                    if constexpr (HAS_Z) y[k] = fmaf(cv[k], h, y[k]);
                }
                // adjoint: lam_t = C_t dy_t + e_t lam_{t+1}, e_t = a_{t+1}.  The last step of
                // lane 63 takes e = 1 and the carry G, which already holds a*lam of the next
                // chunk's first step.
                const float a_next = dpp<kWaveShl1, 0xf>(1.0f, a[0]);
                float cdy[K];
                float r = 0.0f;
#pragma unroll
                for (int k = K - 1; k >= 0; --k) {
                    cdy[k] = cv[k] * dy[k];
                    const float e = (k == K - 1) ? a_next : a[k + 1];
                    r = fmaf(e, r, cdy[k]);
                }
                float Pr = exp2_hw(An2 * (sum_dt - dt[0] + dt_next));
                float Sr = r;
                wave_scan_rev(Pr, Sr);
                float Prx, Srx;
                wave_shift_rev(Pr, Sr, Prx, Srx);
                float lam = fmaf(Prx, readlane(G, n), Srx);
                float dA_part = 0.0f;
#pragma unroll
                for (int k = K - 1; k >= 0; --k) {
                    const float e = (k == K - 1) ? a_next : a[k + 1];
                    lam = fmaf(e, lam, cdy[k]);
                    const float hprev = (k == 0) ? hin : hs[k - 1];
                    const float gk = lam * hprev * a[k];
                    dA_part = fmaf(gk, dt[k], dA_part);
                    sgA[k] = fmaf(gk, An, sgA[k]);
                    sB[k] = fmaf(lam, bv[k], sB[k]);
                    atomicAdd(&accB[buf][k * KP + lane], lam * dtu[k]);
                    atomicAdd(&accC[buf][k * KP + lane], dy[k] * hs[k]);
                }
                G = writelane(readlane(a[0] * lam, 0), n, G);
                accA[wave][n][lane] += dA_part;
            }
            __syncthreads();
            // flush this state's dB/dC tile; the buffer is written again two iterations later,
            // after the next barrier.
            for (int i = tid; i < kChunk; i += 64 * W) {
                const int k = i % K;
                const int ln = i / K;
                const int t = c * kChunk + i;
                const float vb = accB[buf][k * KP + ln];
                const float vc = accC[buf][k * KP + ln];
                accB[buf][k * KP + ln] = 0.0f;
                accC[buf][k * KP + ln] = 0.0f;
                if (t < L) {
                    const size_t o = (static_cast<size_t>(b) * N + n) * L + t;
                    if (g.dB != nullptr) unsafeAtomicAdd(g.dB + o, vb);
                    if (g.dC != nullptr) unsafeAtomicAdd(g.dC + o, vc);
                }
            }
        }

        if (active) {
            float o1[K], o2[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const bool valid = t0 + k < L;
                o1[k] = fmaf(sB[k], dt[k], dy[k] * Dd);               // du
                o2[k] = fmaf(sB[k], uu[k], sgA[k]) * dsp[k];         // ddelta
                dbias_acc += valid ? o2[k] : 0.0f;
            }
            store_k<T, K, VEC>(du_o, t0, L, o1);
            store_k<T, K, VEC>(dd_o, t0, L, o2);
            if constexpr (HAS_Z) {
#pragma unroll
                for (int k = 0; k < K; ++k) o1[k] = gz[k] * y[k];
                store_k<T, K, VEC>(dz_o, t0, L, o1);
            }
        }
    }

    if (active) {
        if (g.dA != nullptr) {
            for (int n = 0; n < N; ++n) {
                const float s = wave_sum(accA[wave][n][lane]);
                if (lane == 0) unsafeAtomicAdd(g.dA + static_cast<size_t>(d) * N + n, s);
            }
        }
        const float sD = wave_sum(dD_acc);
        const float sb = wave_sum(dbias_acc);
        if (lane == 0) {
            if (g.dD != nullptr) unsafeAtomicAdd(g.dD + d, sD);
            if (g.dbias != nullptr) unsafeAtomicAdd(g.dbias + d, sb);
        }
        if (g.dh0 != nullptr && lane < N) g.dh0[ch * N + lane] = G;
    }
}

__global__ void fill_zero_kernel(float* __restrict__ p, size_t n) {
    size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (; i < n; i += stride) p[i] = 0.0f;
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t stream) {
    if (p == nullptr || n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       stream, p, n);
    return hipGetLastError();
}

namespace {

template <typename T, bool VEC, bool HAS_Z, bool SP>
hipError_t bwd_go(const ScanParams& p, const GradParams& g, const float* cst, hipStream_t s) {
    dim3 grid((p.D + kBwdWaves - 1) / kBwdWaves, p.B), block(64 * kBwdWaves);
    hipLaunchKernelGGL((scan_bwd_kernel<T, VEC, HAS_Z, SP>), grid, block, 0, s, p, g, cst);
    return hipGetLastError();
}

template <typename T>
hipError_t bwd_dispatch(const ScanParams& p, const GradParams& g, const float* cst,
                        hipStream_t s) {
    const bool vec = (static_cast<size_t>(p.L) * sizeof(T)) % 16 == 0;
    const bool hz = p.z != nullptr;
    const bool sp = p.softplus != 0;
#define MSEL_BWD(V, Z, S) \
    if (vec == V && hz == Z && sp == S) return bwd_go<T, V, Z, S>(p, g, cst, s);
    MSEL_BWD(true, true, true)
    MSEL_BWD(true, true, false)
    MSEL_BWD(true, false, true)
    MSEL_BWD(true, false, false)
    MSEL_BWD(false, true, true)
    MSEL_BWD(false, true, false)
    MSEL_BWD(false, false, true)
    MSEL_BWD(false, false, false)
#undef MSEL_BWD
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scan_bwd(const ScanParams& p, const GradParams& g, const float* chunk_states,
                           bool bf16, hipStream_t stream) {
    if (p.N > kMaxN) return hipErrorInvalidValue;
    if (bf16) return bwd_dispatch<bf16_t>(p, g, chunk_states, stream);
    return bwd_dispatch<float>(p, g, chunk_states, stream);
}

}  // namespace msel
