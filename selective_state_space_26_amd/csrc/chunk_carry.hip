// chunk_carry.hip -- the chunk-carry pass for gfx950.
//
// Page 4, Appendix D (Speed paragraph): a sequence that does not fit on chip is split into
// chunks, and the scan continues with the next chunk as long as the intermediate state is
// known.  This pass produces exactly those intermediate states.  For each chunk c of
// T = kChunk steps it forms the chunk's transition P_c = exp(A * sum of Delta over the chunk)
// and its local end state S_c (the chunk scanned from a zero state), then links the chunks:
// H_0 = h0, H_{c+1} = P_c H_c + S_c.  H_c goes to chunk_states, H_{n_chunks} to final_state.
//
// One wavefront per (batch, channel); lane l covers steps [c*T + l*K, c*T + (l+1)*K).  Per
// state n the lanes build their own (P, S) pairs and a 64-lane DPP scan composes them into the
// chunk's pair; only the readout is skipped, so it reads u, delta and B but not C or z.
#include "msel_device.hpp"
#include "msel_kernels.hpp"

namespace msel {

template <typename T, bool VEC, bool SOFTPLUS>
__global__ __launch_bounds__(256) void chunk_carry_kernel(ScanParams p) {
    constexpr int K = kChunk / 64;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ch = blockIdx.x * (blockDim.x >> 6) + wave;
    if (ch >= p.B * p.D) return;
    const int b = ch / p.D;
    const int d = ch - b * p.D;
    const int L = p.L;
    const int N = p.N;
    const size_t row = static_cast<size_t>(ch) * L;
    const T* __restrict__ u = static_cast<const T*>(p.u) + row;
    const T* __restrict__ dl = static_cast<const T*>(p.delta) + row;
    const T* __restrict__ Bb = static_cast<const T*>(p.Bm) + static_cast<size_t>(b) * N * L;
    const float bias = p.bias ? p.bias[d] : 0.0f;
    // lane n holds A[d, n] * log2(e): one vector load, read per state with readlane
    const float Av = (lane < N) ? p.A[static_cast<size_t>(d) * N + lane] * kLog2e : 0.0f;
    float* __restrict__ cs = p.chunk_states + static_cast<size_t>(ch) * p.nchunks * N;

    float carry = 0.0f;
    if (p.h0 != nullptr && lane < N) carry = p.h0[static_cast<size_t>(ch) * N + lane];

    for (int c = 0; c < p.nchunks; ++c) {
        if (lane < N) cs[static_cast<size_t>(c) * N + lane] = carry;
        const int t0 = c * kChunk + lane * K;
        float dt[K], du[K];
        float sum_dt = 0.0f;
        {
            float uu[K], dd[K];
            load_k<T, K, VEC>(u, t0, L, uu, 0.0f);
            load_k<T, K, VEC>(dl, t0, L, dd, 0.0f);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float x = dd[k] + bias;
                const float v = SOFTPLUS ? softplus_f(x) : x;
                dt[k] = (t0 + k < L) ? v : 0.0f;
                du[k] = dt[k] * uu[k];
                sum_dt += dt[k];
            }
        }
        Raw<T, K> Bn;
        load_raw<T, K, VEC>(Bb, t0, L, Bn);
        for (int n = 0; n < N; ++n) {
            const float An = readlane(Av, n);
            float bc[K];
            unpack(Bn, bc);
            if (n + 1 < N) load_raw<T, K, VEC>(Bb + static_cast<size_t>(n + 1) * L, t0, L, Bn);
            float h = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k) h = fmaf(exp2_hw(dt[k] * An), h, du[k] * bc[k]);
            float P = exp2_hw(An * sum_dt);
            float S = h;
            scan_fwd_fused(P, S);
            const float cn = readlane(carry, n);
            carry = writelane(readlane(fmaf(P, cn, S), 63), n, carry);
        }
    }
    if (p.final_state != nullptr && lane < N)
        p.final_state[static_cast<size_t>(ch) * N + lane] = carry;
}

namespace {

constexpr int kCcWaves = 4;

template <typename T, bool VEC, bool SP>
hipError_t cc_go(const ScanParams& p, hipStream_t s) {
    const int ch = p.B * p.D;
    dim3 grid((ch + kCcWaves - 1) / kCcWaves), block(64 * kCcWaves);
    hipLaunchKernelGGL((chunk_carry_kernel<T, VEC, SP>), grid, block, 0, s, p);
    return hipGetLastError();
}

template <typename T>
hipError_t cc_dispatch(const ScanParams& p, hipStream_t s) {
    const bool vec = (static_cast<size_t>(p.L) * sizeof(T)) % 16 == 0;
    const bool sp = p.softplus != 0;
    if (vec && sp) return cc_go<T, true, true>(p, s);
    if (vec && !sp) return cc_go<T, true, false>(p, s);
    if (!vec && sp) return cc_go<T, false, true>(p, s);
    return cc_go<T, false, false>(p, s);
}

}  // namespace

hipError_t launch_chunk_carry(const ScanParams& p, bool bf16, hipStream_t stream) {
    if (bf16) return cc_dispatch<bf16_t>(p, stream);
    return cc_dispatch<float>(p, stream);
}

}  // namespace msel
