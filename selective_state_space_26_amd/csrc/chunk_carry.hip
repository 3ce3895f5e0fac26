// chunk_carry.hip -- the chunk-carry pass for gfx950.
//
// Page 4, Appendix D (Speed paragraph): a sequence that does not fit on chip is split into
// chunks, and the scan continues with the next chunk as long as the intermediate state is
// known.  This pass produces exactly those intermediate states.  For each chunk c of
// T = kChunk steps it forms the chunk's transition P_c = exp(A * sum of Delta over the chunk)
// and its local end state S_c (the chunk scanned from a zero state), then links the chunks:
// H_0 = h0, H_{c+1} = P_c H_c + S_c.  H_c goes to chunk_states, H_{n_chunks} to final_state.
//
// Two channels of one batch row per wavefront (each B row read serves both); lane l covers
// steps [c*T + l*K, c*T + (l+1)*K).  Only the chunk totals are needed, so no scan is run: with
// F'_t = the sum of Delta over the chunk's steps after t, the product of a = exp(Delta A) over
// those steps is exp(A F'_t), and
//   S_c = sum_t exp(A F'_t) Delta_t u_t B_t,   P_c = exp(A * the chunk's sum of Delta).
// One suffix sum of Delta per chunk serves all states; every term is independent, and the
// 64-lane sums are done four at a time.  F'_t is summed from the steps it covers (a reversed
// lane scan), not taken as total - prefix: a selective model may reset its state with one
// huge Delta (page 1, the model forgets depending on the current token), and next to it such
// a difference would keep only a few bits of F'_t.  The link runs on all states at once (lane
// n holds state n).  It reads u, delta and B only.
#include "msel_device.hpp"
#include "msel_kernels.hpp"

namespace msel {

constexpr int kCcChannels = 2;  // channels per wavefront: each B row read serves both

template <typename T, bool VEC, bool SOFTPLUS>
__global__ __launch_bounds__(256) void chunk_carry_kernel(ScanParams p) {
    constexpr int K = kChunk / 64;
    constexpr int R = kCcChannels;
    const int lane = lane_id();
    const int rev_addr = (63 - lane) << 2;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int dgroups = (p.D + R - 1) / R;
    const int idx = blockIdx.x * (blockDim.x >> 6) + wave;  // b * dgroups + dg
    if (idx >= p.B * dgroups) return;
    const int b = idx / dgroups;
    const int dg = idx - b * dgroups;
    const int L = p.L;
    const int N = p.N;
    const T* __restrict__ Bb = static_cast<const T*>(p.Bm) + static_cast<size_t>(b) * N * L;

    int dch[R];
    bool live[R];
    const T* u[R];
    const T* dl[R];
    float bias[R], Av[R], carry[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int d = dg * R + r;
        live[r] = d < p.D;
        dch[r] = live[r] ? d : p.D - 1;
        const size_t ch = static_cast<size_t>(b) * p.D + dch[r];
        u[r] = static_cast<const T*>(p.u) + ch * L;
        dl[r] = static_cast<const T*>(p.delta) + ch * L;
        bias[r] = p.bias ? p.bias[dch[r]] : 0.0f;
        // lane n holds A[d, n] * log2(e) and the state h_n entering the current chunk
        Av[r] = (lane < N) ? p.A[static_cast<size_t>(dch[r]) * N + lane] * kLog2e : 0.0f;
        carry[r] = (p.h0 != nullptr && lane < N) ? p.h0[ch * N + lane] : 0.0f;
    }

    for (int c = 0; c < p.nchunks; ++c) {
        const int t0 = c * kChunk + lane * K;
        // F'_t (sum of Delta over the chunk's steps after t), Delta u, and the chunk's total
        float Fs[R][K], du[R][K], total[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (live[r] && lane < N)
                p.chunk_states[((static_cast<size_t>(b) * p.D + dch[r]) * p.nchunks + c) * N +
                               lane] = carry[r];
            float uu[K], dd[K];
            load_k_cached<T, K, VEC>(u[r], t0, L, uu);
            load_k_cached<T, K, VEC>(dl[r], t0, L, dd);
            float dt[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float x = dd[k] + bias[r];
                const float v = SOFTPLUS ? softplus_f(x) : x;
                dt[k] = (t0 + k < L) ? v : 0.0f;
                du[r][k] = dt[k] * uu[k];
            }
            // suffix sums, each a sum of the steps it covers (never total - prefix: next to a
            // reset step's huge Delta that difference would lose the remainder)
            float suf = 0.0f;
#pragma unroll
            for (int k = K - 1; k >= 0; --k) {
                Fs[r][k] = suf;
                suf += dt[k];
            }
            const float after = wave_excl_suffix_sum(suf, rev_addr);  // lanes after this one
            total[r] = readlane(after, 0) + readlane(suf, 0);
#pragma unroll
            for (int k = 0; k < K; ++k) Fs[r][k] += after;
        }
        // local end state of every state from a zero start, two states at a time; lane n
        // collects state n's total
        float S[R];
#pragma unroll
        for (int r = 0; r < R; ++r) S[r] = 0.0f;
        Raw<T, K> B1, B2;
        load_raw<T, K, VEC>(Bb, t0, L, B1);
        load_raw<T, K, VEC>(Bb + static_cast<size_t>(N > 1 ? 1 : 0) * L, t0, L, B2);
        for (int n = 0; n < N; n += 2) {
            const int n2 = (n + 1 < N) ? n + 1 : n;
            float bv1[K], bv2[K];
            unpack(B1, bv1);
            unpack(B2, bv2);
            if (n + 2 < N) {
                load_raw<T, K, VEC>(Bb + static_cast<size_t>(n + 2) * L, t0, L, B1);
                load_raw<T, K, VEC>(Bb + static_cast<size_t>(n + 3 < N ? n + 3 : n + 2) * L, t0,
                                    L, B2);
            }
            float s[4];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float A1 = readlane(Av[r], n), A2 = readlane(Av[r], n2);
                float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    s1 = fmaf(exp2_hw(A1 * Fs[r][k]), du[r][k] * bv1[k], s1);
                    s2 = fmaf(exp2_hw(A2 * Fs[r][k]), du[r][k] * bv2[k], s2);
                }
                s[r] = s1;
                s[2 + r] = s2;
            }
            wave_sum4(s[0], s[1], s[2], s[3]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                S[r] = writelane(s[r], n, S[r]);
                S[r] = writelane(s[2 + r], n2, S[r]);
            }
        }
        // link: H_{c+1} = exp(A * total) H_c + S_c, all states at once (lane n = state n)
#pragma unroll
        for (int r = 0; r < R; ++r) carry[r] = fmaf(exp2_hw(Av[r] * total[r]), carry[r], S[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (p.final_state != nullptr && live[r] && lane < N)
            p.final_state[(static_cast<size_t>(b) * p.D + dch[r]) * N + lane] = carry[r];
}

namespace {

constexpr int kCcWaves = 4;

template <typename T, bool VEC, bool SP>
hipError_t cc_go(const ScanParams& p, hipStream_t s) {
    const int waves = p.B * ((p.D + kCcChannels - 1) / kCcChannels);
    dim3 grid((waves + kCcWaves - 1) / kCcWaves), block(64 * kCcWaves);
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
