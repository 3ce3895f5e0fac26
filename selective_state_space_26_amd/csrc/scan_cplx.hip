// scan_cplx.hip -- fused forward of the complex-valued (rotational) selective scan for gfx950.
//
// Mamba-3 brings back a complex state, written as a scaling and a rotation in a plane so that
// no complex arithmetic type is needed (page 5, the Mamba-3 post, second bullet).  State pair
// (2j, 2j+1) of channel d is one complex state h_j; A[d, 2j] + i A[d, 2j+1] is its rate, and
// rows 2j, 2j+1 of B and C its input and readout:
//
//   a_t = exp(Delta_t A_re) (cos(Delta_t A_im), sin(Delta_t A_im))
//   h_t = a_t h_{t-1} + Delta_t u_t (B_{2j,t}, B_{2j+1,t})         (complex product)
//   y_t = sum_j C_{2j,t} Re h_t + C_{2j+1,t} Im h_t + D u_t,   out_t = y_t silu(z_t)
//
// The layout of the work is the real forward's (scan_fwd.hip): one wavefront per (b, d), tiles
// of 64*K steps, lane l holding K consecutive steps.  Per state pair:
//   pass 1  the lane-local chain of complex affine steps from 0 -> S, and the lane's transition
//           P = exp(A * sum Delta) in closed form (one exp, one sin, one cos);
//   scan    an inclusive 64-lane scan of the complex affine pairs (P, S): per level three
//           copies and eight multiplies and multiply-adds that read the source lane through
//           DPP (a lane without a source keeps its pair: the identity);
//   pass 2  replay from the state entering the lane, y += C . h.
// K steps per lane: 16 for bf16 rows (half the scans per step; 142 VGPRs, 3 wavefronts per
// SIMD), 8 for fp32 rows, whose wider loads of B and C made 16 slower there (86 VGPRs).
// v_sin_f32 / v_cos_f32 take the angle in revolutions; it is reduced to [0, 1) first so that
// any step size stays inside the instructions' input range.
#include "msel_device.hpp"
#include "msel_kernels.hpp"

namespace msel {

namespace {

template <typename T, int K, bool VEC, bool HAS_Z, bool SOFTPLUS>
__global__ __launch_bounds__(256) void scan_cplx_fwd_kernel(ScanParams p) {
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ch = blockIdx.x * (blockDim.x >> 6) + wave;  // b * D + d
    if (ch >= p.B * p.D) return;  // whole wavefront leaves; no barriers here
    const int b = MSEL_IDX(ch / p.D, p.B);
    const int d = ch - b * p.D;
    const int L = p.L;
    const int N = p.N;  // even: N / 2 complex states
    [[maybe_unused]] const size_t BDN = static_cast<size_t>(p.B) * p.D * N;
    const size_t row = static_cast<size_t>(ch) * L;
    const T* __restrict__ u = static_cast<const T*>(p.u) + row;
    const T* __restrict__ dl = static_cast<const T*>(p.delta) + row;
    const T* __restrict__ zr = HAS_Z ? static_cast<const T*>(p.z) + row : nullptr;
    T* __restrict__ out = static_cast<T*>(p.out) + row;
    const T* __restrict__ Bb = static_cast<const T*>(p.Bm) + static_cast<size_t>(b) * N * L;
    const T* __restrict__ Cb = static_cast<const T*>(p.Cm) + static_cast<size_t>(b) * N * L;
    const float bias = p.bias ? p.bias[MSEL_IDX(d, p.D)] : 0.0f;
    const float Dd = p.Dv ? p.Dv[MSEL_IDX(d, p.D)] : 0.0f;
    constexpr int TILE = 64 * K;
    static_assert(TILE % kChunk == 0, "a tile must hold whole chunks");
    constexpr int kCpt = TILE / kChunk;
    // Per wavefront, one float per state component: A (row 0; component 2j: A_re * log2(e)
    // for exp2, 2j+1: A_im / (2 pi) in revolutions), the state entering the tile (row 1) and
    // the states entering the tile's chunks (rows 2 ..).  Read by address (broadcast LDS reads)
    // and written by the one lane that has the value, instead of v_readlane / v_writelane.
    __shared__ float cells[4][2 + kCpt][kMaxN];
    float* const cA = cells[wave][0];
    float* const cH = cells[wave][1];
    if (lane < N) {
        const float a = p.A[MSEL_IDX(static_cast<size_t>(d) * N + lane, static_cast<size_t>(p.D) * N)];
        cA[lane] = (lane & 1) ? a * kInv2Pi : a * kLog2e;
        cH[lane] = p.h0 != nullptr ? p.h0[MSEL_IDX(static_cast<size_t>(ch) * N + lane, BDN)] : 0.0f;
    }

    for (int tile = 0; tile < L; tile += TILE) {
        const int t0 = tile + lane * K;
        float dt[K], du[K], y[K];
        float sum_dt = 0.0f;
        {
            float uu[K], dd[K];
            load_k_cached<T, K, VEC>(u, t0, L, uu);
            load_k_cached<T, K, VEC>(dl, t0, L, dd);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float x = dd[k] + bias;
                const float v = SOFTPLUS ? softplus_f(x) : x;
                dt[k] = (t0 + k < L) ? v : 0.0f;  // Delta = 0 past the end: identity step
                du[k] = dt[k] * uu[k];
                y[k] = Dd * uu[k];
                sum_dt += dt[k];
            }
        }
        for (int n = 0; n < N; n += 2) {
            const float Ar = cA[MSEL_IDX(n, kMaxN - 1)], Ai = cA[MSEL_IDX(n, kMaxN - 1) + 1];
            // the state entering the tile, read early: used right after the scan
            const float cr = cH[MSEL_IDX(n, kMaxN - 1)], ci = cH[MSEL_IDX(n, kMaxN - 1) + 1];
            float ar[K], ai[K], p1[K], p2[K];
            // the pair's C rows are loaded with its B rows and used after the scan, so that
            // their loads are in flight during the chain and the scan
            Raw<T, K> rc1, rc2;
            load_raw<T, K, VEC>(Cb + static_cast<size_t>(MSEL_IDX(n, N)) * L, t0, L, rc1);
            load_raw<T, K, VEC>(Cb + static_cast<size_t>(MSEL_IDX(n + 1, N)) * L, t0, L, rc2);
            load_k_cached<T, K, VEC>(Bb + static_cast<size_t>(MSEL_IDX(n, N)) * L, t0, L, p1);
            load_k_cached<T, K, VEC>(Bb + static_cast<size_t>(MSEL_IDX(n + 1, N)) * L, t0, L, p2);
            float h1 = 0.0f, h2 = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float e = exp2_hw(dt[k] * Ar);
                const float r = dt[k] * Ai;
                ar[k] = e * cos_rev(r);
                ai[k] = e * sin_rev(r);
                p1[k] *= du[k];
                p2[k] *= du[k];
                const float n1 = fmaf(ar[k], h1, fmaf(-ai[k], h2, p1[k]));
                h2 = fmaf(ai[k], h1, fmaf(ar[k], h2, p2[k]));
                h1 = n1;
            }
            const float e = exp2_hw(sum_dt * Ar);
            const float r = sum_dt * Ai;
            float Pr = e * cos_rev(r), Pi = e * sin_rev(r), Sr = h1, Si = h2;
            cscan_fused(Pr, Pi, Sr, Si);
            // state after the lane's last step, and the state entering the lane
            const float Qr = fmaf(Pr, cr, fmaf(-Pi, ci, Sr));
            const float Qi = fmaf(Pr, ci, fmaf(Pi, cr, Si));
            const float hr = shift_up(Qr, cr), hi = shift_up(Qi, ci);
            if (lane == 63) {
                cH[MSEL_IDX(n, kMaxN - 1)] = Qr;
                cH[MSEL_IDX(n, kMaxN - 1) + 1] = Qi;
            }
            if (lane % (kChunk / K) == 0) {  // the first lane of a chunk
                float* cs = cells[wave][MSEL_IDX(2 + lane / (kChunk / K), 2 + kCpt)];
                cs[MSEL_IDX(n, kMaxN - 1)] = hr;
                cs[MSEL_IDX(n, kMaxN - 1) + 1] = hi;
            }

            float c1[K], c2[K];
            unpack(rc1, c1);
            unpack(rc2, c2);
            h1 = hr;
            h2 = hi;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float n1 = fmaf(ar[k], h1, fmaf(-ai[k], h2, p1[k]));
                h2 = fmaf(ai[k], h1, fmaf(ar[k], h2, p2[k]));
                h1 = n1;
                y[k] = fmaf(c1[k], h1, fmaf(c2[k], h2, y[k]));
            }
        }
        if constexpr (HAS_Z) {
            float zz[K];
            load_k_cached<T, K, VEC>(zr, t0, L, zz);
#pragma unroll
            for (int k = 0; k < K; ++k) y[k] *= zz[k] * sigmoid_f(zz[k]);
        }
        store_k<T, K, VEC, false>(out, t0, L, y);
        if (p.chunk_states != nullptr && lane < N) {
#pragma unroll
            for (int q = 0; q < kCpt; ++q) {
                const int cidx = tile / kChunk + q;
                if (cidx < p.nchunks)
                    p.chunk_states[MSEL_IDX((static_cast<size_t>(ch) * p.nchunks + cidx) * N + lane,
                                            BDN * p.nchunks)] = cells[wave][2 + q][lane];
            }
        }
    }
    if (p.final_state != nullptr && lane < N)
        p.final_state[MSEL_IDX(static_cast<size_t>(ch) * N + lane, BDN)] = cH[lane];
}

// The recurrent (decode) step: a 16-lane row per channel, lane n for state component n.  Each
// lane reads both components of its pair (its own and lane n ^ 1's) before any lane writes,
// so final_state may be h0 itself.
template <typename T, bool HAS_Z, bool SOFTPLUS>
__global__ __launch_bounds__(256) void scan_cplx_step_kernel(ScanParams p) {
    const int lane = lane_id();
    const int n = lane & 15;
    // b * D + d, formed in 64 bits: 16 * batch * dim threads may pass 2^32
    const long long ch =
        (static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x) >> 4;
    const long long BD = static_cast<long long>(p.B) * p.D;
    const bool in = ch < BD;
    const int chc = MSEL_IDX(in ? static_cast<int>(ch) : 0, BD);
    const int b = chc / p.D;
    const int d = chc - b * p.D;
    const int N = p.N;
    const bool st = in && n < N;
    const int ne = (n < N ? n : N - 1) & ~1;  // the pair's real component
    [[maybe_unused]] const size_t BN = static_cast<size_t>(p.B) * N;
    [[maybe_unused]] const size_t BDN = static_cast<size_t>(BD) * N;
    const float u = Elem<T>::load1(static_cast<const T*>(p.u) + chc);
    const float x = Elem<T>::load1(static_cast<const T*>(p.delta) + chc) +
                    (p.bias ? p.bias[MSEL_IDX(d, p.D)] : 0.0f);
    const float dt = SOFTPLUS ? softplus_f(x) : x;
    const size_t bn = static_cast<size_t>(b) * N + ne;  // B and C are [batch, dstate, 1]
    // the pair's two components: bn and bn + 1
    const float Br = Elem<T>::load1(static_cast<const T*>(p.Bm) + MSEL_IDX(bn, BN - 1));
    const float Bi = Elem<T>::load1(static_cast<const T*>(p.Bm) + MSEL_IDX(bn, BN - 1) + 1);
    const float Cv = Elem<T>::load1(static_cast<const T*>(p.Cm) + MSEL_IDX(bn, BN - 1) + (n & 1));
    // the pair's A_re and A_im: Ad[0], Ad[1]
    const float* Ad = p.A + static_cast<size_t>(MSEL_IDX(d, p.D)) * N + MSEL_IDX(ne, N - 1);
    const float e = exp2_hw(dt * Ad[0] * kLog2e);
    const float r = dt * Ad[1] * kInv2Pi;
    const float ar = e * cos_rev(r), ai = e * sin_rev(r);
    const size_t sidx = static_cast<size_t>(chc) * N + ne;
    const float h0r = p.h0 ? p.h0[MSEL_IDX(sidx, BDN)] : 0.0f;
    const float h0i = p.h0 ? p.h0[MSEL_IDX(sidx + 1, BDN)] : 0.0f;
    const float h = (n & 1) ? fmaf(ai, h0r, fmaf(ar, h0i, dt * u * Bi))
                            : fmaf(ar, h0r, fmaf(-ai, h0i, dt * u * Br));
    float part = st ? Cv * h : 0.0f;
    // sum over the row's 16 lanes: inclusive DPP prefix, lane 15 of the row holds the total
    asm volatile("s_nop 1\n"
                 "v_add_f32_dpp %[v], %[v], %[v] row_shr:1 row_mask:0xf bank_mask:0xf\n"
                 "s_nop 1\n"
                 "v_add_f32_dpp %[v], %[v], %[v] row_shr:2 row_mask:0xf bank_mask:0xf\n"
                 "s_nop 1\n"
                 "v_add_f32_dpp %[v], %[v], %[v] row_shr:4 row_mask:0xf bank_mask:0xf\n"
                 "s_nop 1\n"
                 "v_add_f32_dpp %[v], %[v], %[v] row_shr:8 row_mask:0xf bank_mask:0xf\n"
                 : [v] "+v"(part));
    if (st) {
        const size_t own = MSEL_IDX(static_cast<size_t>(chc) * N + n, BDN);
        if (p.chunk_states != nullptr) p.chunk_states[own] = (n & 1) ? h0i : h0r;
        if (p.final_state != nullptr) p.final_state[own] = h;
    }
    if (in && n == 15) {
        float yv = part + (p.Dv ? p.Dv[MSEL_IDX(d, p.D)] : 0.0f) * u;
        if constexpr (HAS_Z) {
            const float z = Elem<T>::load1(static_cast<const T*>(p.z) + chc);
            yv *= z * sigmoid_f(z);
        }
        Elem<T>::store1(static_cast<T*>(p.out) + chc, yv);
    }
}

constexpr int kWaves = 4;

template <typename T, bool VEC, bool HAS_Z, bool SP>
hipError_t cplx_go(const ScanParams& p, hipStream_t s) {
    if (p.L == 1) {
        const long long threads = static_cast<long long>(p.B) * p.D * 16;
        hipLaunchKernelGGL((scan_cplx_step_kernel<T, HAS_Z, SP>),
                           dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, s, p);
        return hipGetLastError();
    }
    const int ch = p.B * p.D;
    constexpr int K = sizeof(T) == 2 ? 16 : 8;
    hipLaunchKernelGGL((scan_cplx_fwd_kernel<T, K, VEC, HAS_Z, SP>),
                       dim3((ch + kWaves - 1) / kWaves), dim3(64 * kWaves), 0, s, p);
    return hipGetLastError();
}

template <typename T>
hipError_t cplx_dispatch(const ScanParams& p, hipStream_t s) {
    const bool vec = (static_cast<size_t>(p.L) * sizeof(T)) % 16 == 0;
    const bool hz = p.z != nullptr, sp = p.softplus != 0;
#define MSEL_CPLX(V, Z, S) \
    if (vec == V && hz == Z && sp == S) return cplx_go<T, V, Z, S>(p, s);
    MSEL_CPLX(true, true, true)
    MSEL_CPLX(true, true, false)
    MSEL_CPLX(true, false, true)
    MSEL_CPLX(true, false, false)
    MSEL_CPLX(false, true, true)
    MSEL_CPLX(false, true, false)
    MSEL_CPLX(false, false, true)
    MSEL_CPLX(false, false, false)
#undef MSEL_CPLX
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scan_cplx_fwd(const ScanParams& p, bool bf16, hipStream_t stream) {
    return bf16 ? cplx_dispatch<bf16_t>(p, stream) : cplx_dispatch<float>(p, stream);
}

MSEL_BOUNDS_TAKER(take_bounds_cplx)

}  // namespace msel
