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
//
// The same pass for the two Mamba-3 variants (page 5, the Mamba-3 post):
//  * TRAP, the exponential-trapezoidal rule h_t = a_t (h_{t-1} + c_t B_{t-1}) + g_t u_t B_t
//    with g_t = lambda_t Delta_t and c_t = (1 - lambda_t) Delta_t u_{t-1}.  Step t's input
//    reaches back to step t-1's B, so, summed over the chunk,
//      S_c = sum_t exp(A F'_t) B_t (g_t u_t + c_{t+1})      (c_{t+1} = 0 at the chunk's end)
//    and the term of the chunk's first step that reaches into the previous chunk joins the
//    link: H_{c+1} = P_c (H_c + c_{t0} B_{t0-1}) + S_c, with B_{t0-1}, u_{t0-1} the previous
//    chunk's last step (u_prev, B_prev before the first chunk).  It also reads lambda.
//  * CPLX, the complex-valued state: pairs (2j, 2j+1) are one complex state with the complex
//    rate A[d, 2j] + i A[d, 2j+1]; exp(A F') is a scaling and a rotation, the input is
//    Delta u (B_2j + i B_2j+1), and the link multiplies complex numbers across the pair's two
//    lanes.
#include "msel_device.hpp"
#include "msel_kernels.hpp"

namespace msel {

constexpr int kCcChannels = 2;  // channels per wavefront: each B row read serves both

enum class CcRule { kPlain, kTrap, kCplx };

template <typename T, bool VEC, bool SOFTPLUS, CcRule RULE>
__global__ __launch_bounds__(256) void chunk_carry_kernel(ScanParams p) {
    constexpr int K = kChunk / 64;
    constexpr int R = kCcChannels;
    constexpr bool TRAP = RULE == CcRule::kTrap;
    constexpr bool CPLX = RULE == CcRule::kCplx;
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
    const T* __restrict__ Bb =
        static_cast<const T*>(p.Bm) + static_cast<size_t>(MSEL_IDX(b, p.B)) * N * L;
    [[maybe_unused]] const size_t BDN = static_cast<size_t>(p.B) * p.D * N;

    int dch[R];
    bool live[R];
    const T* u[R];
    const T* dl[R];
    const T* lm[R];
    float bias[R], Av[R], carry[R];
    float u_last[R];    // TRAP: u at the step before the current chunk (wave-uniform)
    float Are[R], Aim[R];  // CPLX: the rate of lane n's pair, A_re log2(e) and A_im / (2 pi)
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int d = dg * R + r;
        live[r] = d < p.D;
        dch[r] = live[r] ? d : p.D - 1;
        const size_t ch = MSEL_IDX(static_cast<size_t>(b) * p.D + dch[r],
                                   static_cast<size_t>(p.B) * p.D);
        u[r] = static_cast<const T*>(p.u) + ch * L;
        dl[r] = static_cast<const T*>(p.delta) + ch * L;
        lm[r] = TRAP ? static_cast<const T*>(p.lam) + ch * L : nullptr;
        bias[r] = p.bias ? p.bias[MSEL_IDX(dch[r], p.D)] : 0.0f;
        const float* Ad = p.A + static_cast<size_t>(MSEL_IDX(dch[r], p.D)) * N;
        // lane n holds A[d, n] * log2(e) (CPLX: lane 2j+1 holds A_im / (2 pi), in revolutions)
        // and the state h_n entering the current chunk
        if constexpr (CPLX) {
            Av[r] = (lane < N) ? ((lane & 1) ? Ad[MSEL_IDX(lane, N)] * kInv2Pi
                                             : Ad[MSEL_IDX(lane, N)] * kLog2e)
                               : 0.0f;
            Are[r] = (lane < N) ? Ad[MSEL_IDX(lane & ~1, N)] * kLog2e : 0.0f;
            Aim[r] = (lane < N) ? Ad[MSEL_IDX(lane | 1, N)] * kInv2Pi : 0.0f;
        } else {
            Av[r] = (lane < N) ? Ad[MSEL_IDX(lane < N ? lane : 0, N)] * kLog2e : 0.0f;
        }
        carry[r] = (p.h0 != nullptr && lane < N) ? p.h0[MSEL_IDX(ch * N + lane, BDN)] : 0.0f;
        u_last[r] = 0.0f;
        if constexpr (TRAP)
            if (p.u_prev != nullptr) u_last[r] = Elem<T>::load1(static_cast<const T*>(p.u_prev) + ch);
    }
    // TRAP: lane n holds B of state n at the step before the current chunk
    float B_last = 0.0f;
    if constexpr (TRAP)
        if (p.B_prev != nullptr && lane < N)
            B_last = Elem<T>::load1(static_cast<const T*>(p.B_prev) +
                                    MSEL_IDX(static_cast<size_t>(b) * N + lane,
                                             static_cast<size_t>(p.B) * N));

    // each chunk's u, delta (TRAP: lambda) rows are loaded while the chunk before is computed
    Raw<T, K> ru[R], rd[R], rl[TRAP ? R : 1];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        load_raw<T, K, VEC>(u[r], lane * K, L, ru[r]);
        load_raw<T, K, VEC>(dl[r], lane * K, L, rd[r]);
        if constexpr (TRAP) load_raw<T, K, VEC>(lm[r], lane * K, L, rl[r]);
    }
    // the first pair of B rows of each chunk is loaded during the chunk before
    Raw<T, K> B1, B2;
    load_raw<T, K, VEC>(Bb, lane * K, L, B1);
    load_raw<T, K, VEC>(Bb + static_cast<size_t>(MSEL_IDX(N > 1 ? 1 : 0, N)) * L, lane * K, L, B2);
    for (int c = 0; c < p.nchunks; ++c) {
        const int t0 = c * kChunk + lane * K;
        // the next chunk's rows; after the last chunk past the row's end (zeros, no access)
        const int tn = (c + 1 < p.nchunks) ? t0 + kChunk : L;
        // F'_t (sum of Delta over the chunk's steps after t), each step's input weight w_t
        // (Delta u; TRAP: g u + c_{t+1}), and the chunk's total
        float Fs[R][K], w[R][K], total[R];
        float cb[R];  // TRAP: c at the chunk's first step (wave-uniform)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (live[r] && lane < N)
                p.chunk_states[MSEL_IDX(
                    ((static_cast<size_t>(b) * p.D + dch[r]) * p.nchunks + c) * N + lane,
                    BDN * p.nchunks)] = carry[r];
            float uu[K], dd[K], ll[TRAP ? K : 1];
            unpack(ru[r], uu);
            unpack(rd[r], dd);
            if constexpr (TRAP) unpack(rl[r], ll);
            load_raw<T, K, VEC>(u[r], tn, L, ru[r]);
            load_raw<T, K, VEC>(dl[r], tn, L, rd[r]);
            if constexpr (TRAP) load_raw<T, K, VEC>(lm[r], tn, L, rl[r]);
            float dt[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float x = dd[k] + bias[r];
                const float v = SOFTPLUS ? softplus_f(x) : x;
                dt[k] = (t0 + k < L) ? v : 0.0f;
            }
            if constexpr (TRAP) {
                float cp[K];  // c_t = (1 - lambda_t) Delta_t u_{t-1}
                const float um1_0 = shift_up(uu[K - 1], u_last[r]);
#pragma unroll
                for (int k = 0; k < K; ++k)
                    cp[k] = (dt[k] - ll[k] * dt[k]) * (k == 0 ? um1_0 : uu[k - 1]);
                const float cnext = shift_down(cp[0], 0.0f);  // lane 63: the next chunk's
#pragma unroll
                for (int k = 0; k < K; ++k)
                    w[r][k] = fmaf(ll[k] * dt[k], uu[k], k + 1 < K ? cp[k + 1] : cnext);
                cb[r] = readlane(cp[0], 0);
                u_last[r] = readlane(uu[K - 1], 63);
            } else {
#pragma unroll
                for (int k = 0; k < K; ++k) w[r][k] = dt[k] * uu[k];
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
        // local end state of every state from a zero start, two states at a time (CPLX: one
        // complex state, the pair (n, n+1)); lane n collects state n's total
        float S[R];
#pragma unroll
        for (int r = 0; r < R; ++r) S[r] = 0.0f;
        float B_next = B_last;  // TRAP: B of every state at this chunk's last step
        for (int n = 0; n < N; n += 2) {
            const int n2 = (n + 1 < N) ? n + 1 : n;
            float bv1[K], bv2[K];
            unpack(B1, bv1);
            unpack(B2, bv2);
            {
                // the next pair's rows: of this chunk, or after the last pair the next chunk's
                // first (past the row's end after the last chunk: zeros, no access)
                const bool in = n + 2 < N;
                const int na = in ? n + 2 : 0;
                const int nb = in ? (n + 3 < N ? n + 3 : n + 2) : (N > 1 ? 1 : 0);
                const int tb = in ? t0 : tn;
                load_raw<T, K, VEC>(Bb + static_cast<size_t>(MSEL_IDX(na, N)) * L, tb, L, B1);
                load_raw<T, K, VEC>(Bb + static_cast<size_t>(MSEL_IDX(nb, N)) * L, tb, L, B2);
            }
            if constexpr (TRAP) {
                B_next = writelane(readlane(bv1[K - 1], 63), n, B_next);
                B_next = writelane(readlane(bv2[K - 1], 63), n2, B_next);
            }
            float s[4];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float A1 = readlane(Av[r], n), A2 = readlane(Av[r], n2);
                float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    if constexpr (CPLX) {
                        // exp(A F') (Delta u)(B_n + i B_n2): scaling, rotation, complex input
                        const float e = exp2_hw(A1 * Fs[r][k]);
                        const float th = A2 * Fs[r][k];
                        const float co = e * cos_rev(th), si = e * sin_rev(th);
                        const float pr = w[r][k] * bv1[k], pi = w[r][k] * bv2[k];
                        s1 = fmaf(co, pr, fmaf(-si, pi, s1));
                        s2 = fmaf(si, pr, fmaf(co, pi, s2));
                    } else {
                        s1 = fmaf(exp2_hw(A1 * Fs[r][k]), w[r][k] * bv1[k], s1);
                        s2 = fmaf(exp2_hw(A2 * Fs[r][k]), w[r][k] * bv2[k], s2);
                    }
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
        // link: H_{c+1} = P_c H_c + S_c, all states at once (lane n = state n)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if constexpr (CPLX) {
                // P_c = exp(A total) as a complex number; lane 2j holds Re, 2j+1 Im:
                // Re' = Pr Re - Pi Im, Im' = Pr Im + Pi Re
                const float e = exp2_hw(Are[r] * total[r]);
                const float th = Aim[r] * total[r];
                const float pr = e * cos_rev(th), pi = e * sin_rev(th);
                const float other = dpp<0xB1, 0xf>(0.0f, carry[r]);  // the pair's other part
                carry[r] = fmaf(pr, carry[r], fmaf((lane & 1) ? pi : -pi, other, S[r]));
            } else if constexpr (TRAP) {
                carry[r] = fmaf(exp2_hw(Av[r] * total[r]), fmaf(cb[r], B_last, carry[r]), S[r]);
            } else {
                carry[r] = fmaf(exp2_hw(Av[r] * total[r]), carry[r], S[r]);
            }
        }
        if constexpr (TRAP) B_last = B_next;
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (p.final_state != nullptr && live[r] && lane < N)
            p.final_state[MSEL_IDX((static_cast<size_t>(b) * p.D + dch[r]) * N + lane, BDN)] =
                carry[r];
}

namespace {

constexpr int kCcWaves = 4;

template <typename T, bool VEC, bool SP, CcRule RULE>
hipError_t cc_go(const ScanParams& p, hipStream_t s) {
    const int waves = p.B * ((p.D + kCcChannels - 1) / kCcChannels);
    dim3 grid((waves + kCcWaves - 1) / kCcWaves), block(64 * kCcWaves);
    hipLaunchKernelGGL((chunk_carry_kernel<T, VEC, SP, RULE>), grid, block, 0, s, p);
    return hipGetLastError();
}

template <typename T, CcRule RULE>
hipError_t cc_dispatch(const ScanParams& p, hipStream_t s) {
    const bool vec = (static_cast<size_t>(p.L) * sizeof(T)) % 16 == 0;
    const bool sp = p.softplus != 0;
    if (vec && sp) return cc_go<T, true, true, RULE>(p, s);
    if (vec && !sp) return cc_go<T, true, false, RULE>(p, s);
    if (!vec && sp) return cc_go<T, false, true, RULE>(p, s);
    return cc_go<T, false, false, RULE>(p, s);
}

template <typename T>
hipError_t cc_rule(const ScanParams& p, bool cplx, hipStream_t s) {
    if (cplx) return cc_dispatch<T, CcRule::kCplx>(p, s);
    if (p.lam != nullptr) return cc_dispatch<T, CcRule::kTrap>(p, s);
    return cc_dispatch<T, CcRule::kPlain>(p, s);
}

}  // namespace

hipError_t launch_chunk_carry(const ScanParams& p, bool bf16, bool cplx, hipStream_t stream) {
    if (bf16) return cc_rule<bf16_t>(p, cplx, stream);
    return cc_rule<float>(p, cplx, stream);
}

MSEL_BOUNDS_TAKER(take_bounds_chunk_carry)

}  // namespace msel
