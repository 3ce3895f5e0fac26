// scan_fwd.hip -- fused forward selective scan for gfx950.
//
// One wavefront owns one (batch, channel) recurrence and walks the sequence in tiles of
// 64*K time steps; lane l holds the K consecutive steps [tile + l*K, tile + (l+1)*K).  The
// scan is fused in one pass over HBM (page 4, Appendix D, Speed paragraph: memory-bound
// operations are fused so that u, Delta, B, C, z are read once and only out is written):
//
//   per tile: load u, delta (and later z) for the lane's K steps, Delta = softplus(delta+bias),
//   per state n:
//     pass 1  a_k = exp2(Delta_k * A'_n)           (A' = A*log2 e: ZOH transition)
//             b_k = Delta_k u_k * B_{n,k}           (Euler input)
//             lane-local chain from 0 -> S, and P = exp2(A'_n * sum Delta) (lane transition)
//     scan    inclusive DPP scan of (P, S) over the 64 lanes (DPP fused into the fma/mul),
//             applied to the state carried from the previous tile and shifted by one lane ->
//             state entering the lane (page 1: the recurrence is parallelized with a
//             work-efficient scan)
//     pass 2  replay the chain from that state, y_k += C_{n,k} h_k
//   epilogue: y += D u (initialised up front), out = y * silu(z), one store.
//
// A workgroup holds four channels of one batch row, which share B and C: their rows of each
// state are read (and, in bf16, converted to fp32) once per workgroup into a double-buffered
// LDS stage (see the kernel) and read from there by every wavefront.
//
// The state never leaves the chip: the carried state of all N states lives in the
// wavefront's LDS cells (one float per state), so long sequences are handled by the tile loop
// with the state carried across tiles (page 4, Appendix D: split the sequence into chunks,
// continue the scan from the intermediate state).  Lanes at multiples of the chunk length also
// write the state entering them to chunk_states.
//
// TRAP: the exponential-trapezoidal rule of Mamba-3 (page 5, first bullet: the input integral
// over a step taken from both ends of the interval, mixed by a data-dependent weight lambda):
//   b_k = a_k * ((1 - lambda_k) Delta_k u_{k-1}) * B_{n,k-1} + (lambda_k Delta_k u_k) * B_{n,k}
// The step-(k-1) factors come from the lane's own registers, from lane l-1 for its first step
// (a DPP shift), and from the previous tile's last step (u wave-uniform, B of state n in lane
// n of one VGPR) or u_prev / B_prev for the first tile.  The transition a_k, the lane
// transition P and everything after pass 1 are unchanged.
#include "msel_device.hpp"
#include "msel_kernels.hpp"

namespace msel {

// Channels of one batch row per workgroup: with the stage (below), the more share it, the
// fewer conversions and L2 reads of B and C per channel.  (8 and 16 were slower: each state
// then waits at a wider barrier.)
constexpr int kFwdStageWaves = 4;
template <typename T, bool TRAP>
__host__ __device__ constexpr int fwd_waves() { return !TRAP ? kFwdStageWaves : 4; }

// STAGE (plain rule): a state's B and C rows over a tile are read from L2 once per workgroup
// (bf16 converted to fp32 on the way), into LDS, and read by each of its wavefronts, instead
// of by every wavefront: [2 tensors][K/4 words][64 lanes + 2] of 16-byte words, so that a
// lane's K steps are K/4 words of its own column and the 64 lanes read consecutive words.  Two
// buffers: the next state's rows are staged while the current one is computed, with one
// barrier per state.  Without the stage an fp32 wavefront streams 8 KB of B and C rows per
// state and tile through L2, eight times the HBM bytes it reads.  (The trapezoidal rule loads
// B and C per wavefront: with the stage it needs 143 VGPRs, 3 wavefronts per SIMD, and ran
// slower.)
template <typename T, int K, bool VEC, bool HAS_Z, bool SOFTPLUS, bool TRAP>
__global__ __launch_bounds__((64 * fwd_waves<T, TRAP>())) void scan_fwd_kernel(ScanParams p) {
    constexpr bool STAGE = !TRAP;
    constexpr int kFwdWaves = fwd_waves<T, TRAP>();
    // HALVES (bf16 rows of whole vectors): the two halves of the workgroup stage the states
    // in turn (below)
    constexpr bool HALVES = STAGE && sizeof(T) == 2 && VEC;
    using Stage = TileStage<T, K, 2, (HALVES ? 32 : 64) * kFwdWaves, VEC>;  // rows: B, C
    __shared__ f32x4 stage[STAGE ? 2 : 1][STAGE ? Stage::kWords : 1];
    // Per wavefront, one float per state: A' (row 0), the state carried into the tile (row
    // 1) and the states entering the tile's chunks (rows 2 ..).  A state's value is read by
    // address (one broadcast LDS read) and written by the one lane that has it, instead of a
    // v_readlane / v_writelane per state.
    constexpr int kCpt = 64 * K / kChunk;  // chunks per tile
    __shared__ float cells[kFwdWaves][2 + kCpt][kMaxN];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // one-dimensional grid over (batch row, group of channels), channel groups fastest
    const int ngrp = (p.D + kFwdWaves - 1) / kFwdWaves;
    const int b = static_cast<int>(blockIdx.x) / ngrp;
    const int dw = (static_cast<int>(blockIdx.x) - b * ngrp) * kFwdWaves + wave;
    // wave-uniform.  Without the stage a wavefront past the last channel leaves (no barriers
    // then); with it, it computes channel D-1 again (its addresses stay valid), takes part in
    // the staging and the barriers, and stores nothing.
    const bool active = dw < p.D;
    if (!STAGE && !active) return;
    const int d = active ? dw : p.D - 1;
    const int ch = MSEL_IDX(b * p.D + d, static_cast<long long>(p.B) * p.D);
    const int L = p.L;
    const int N = p.N;
    const size_t row = static_cast<size_t>(ch) * L;
    const T* __restrict__ u = static_cast<const T*>(p.u) + row;
    const T* __restrict__ dl = static_cast<const T*>(p.delta) + row;
    const T* __restrict__ zr = HAS_Z ? static_cast<const T*>(p.z) + row : nullptr;
    T* __restrict__ out = static_cast<T*>(p.out) + row;
    const T* __restrict__ Bb =
        static_cast<const T*>(p.Bm) + static_cast<size_t>(MSEL_IDX(b, p.B)) * N * L;
    const T* __restrict__ Cb =
        static_cast<const T*>(p.Cm) + static_cast<size_t>(MSEL_IDX(b, p.B)) * N * L;
    const float bias = p.bias ? p.bias[MSEL_IDX(d, p.D)] : 0.0f;
    const float Dd = p.Dv ? p.Dv[MSEL_IDX(d, p.D)] : 0.0f;
    [[maybe_unused]] const size_t DN = static_cast<size_t>(p.D) * N;
    [[maybe_unused]] const size_t BDN = static_cast<size_t>(p.B) * DN;
    // A[d, n] * log2(e) and the state h_n entering the current tile, from lane n
    float* const cA = cells[wave][0];
    float* const cH = cells[wave][1];
    if (lane < N) {
        cA[lane] = p.A[MSEL_IDX(static_cast<size_t>(d) * N + lane, DN)] * kLog2e;
        cH[lane] = p.h0 != nullptr ? p.h0[MSEL_IDX(static_cast<size_t>(ch) * N + lane, BDN)]
                                   : 0.0f;
    }
    // TRAP: the step before the tile: its u (wave-uniform) and B (lane n: state n)
    float u_last = 0.0f, B_last = 0.0f;
    if constexpr (TRAP) {
        if (p.u_prev != nullptr) u_last = Elem<T>::load1(static_cast<const T*>(p.u_prev) + ch);
        if (p.B_prev != nullptr && lane < N)
            B_last = Elem<T>::load1(static_cast<const T*>(p.B_prev) +
                                    MSEL_IDX(static_cast<size_t>(b) * N + lane,
                                             static_cast<size_t>(p.B) * N));
    }

    constexpr int TILE = 64 * K;
    static_assert(TILE % kChunk == 0, "a tile must hold whole chunks");

    // Each state's rows are loaded while the state before it is computed and staged at its
    // end.  HALVES: the two halves of the workgroup (wavefronts 0, 2 and 1, 3) stage the
    // states in turn, by the parity of a state's place g in the walk over all tiles: a half
    // loads a state's rows at the start of the state two before it and stages them at the end
    // of the state just before it, so that the loads have two states' work to arrive in, with
    // one set of loads in flight per thread.  (In fp32 a thread's share of a state is twice
    // the registers, and the kernel would no longer fit four wavefronts per SIMD.)
    const int par = wave & 1;
    const int stid = HALVES ? (wave >> 1) * 64 + lane : tid;  // the thread's place in its stager
    Stage st(stid);
    auto rows = [&](int n) {  // staged row x of state n: B (x = 0) or C (x = 1)
        return [=](int x) {
            return (x == 0 ? Bb : Cb) + static_cast<size_t>(MSEL_IDX(n, N)) * L;
        };
    };
    int buf = 0;
    int g = 0;  // the current state's place in the walk (wave-uniform)
    if constexpr (STAGE) {
        if (!HALVES || par == 0) {
            st.load(stid, rows(0), 0, L);
            st.store(stid, stage[0]);
        } else if (N > 1 || TILE < L) {  // the second state of the walk
            st.load(stid, rows(N > 1 ? 1 : 0), N > 1 ? 0 : TILE, L);
        }
        __syncthreads();
    }

    for (int tile = 0; tile < L; tile += TILE) {
        const int t0 = tile + lane * K;
        float dt[K], du[K], y[K];
        float cp[TRAP ? K : 1];  // TRAP: (1 - lambda_k) Delta_k u_{k-1}
        float sum_dt = 0.0f;
        {
            float uu[K], dd[K];
            load_k_cached<T, K, VEC>(u, t0, L, uu);
            load_k_cached<T, K, VEC>(dl, t0, L, dd);
            float lm[TRAP ? K : 1];
            if constexpr (TRAP)
                load_k_cached<T, K, VEC>(static_cast<const T*>(p.lam) + row, t0, L, lm);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float x = dd[k] + bias;
                dt[k] = SOFTPLUS ? softplus_f(x) : x;
            }
            if (tile + TILE > L) {  // Delta = 0 past the end: identity steps
#pragma unroll
                for (int k = 0; k < K; ++k) dt[k] = (t0 + k < L) ? dt[k] : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < K; ++k) {
                if constexpr (TRAP) {
                    const float um1 = k == 0 ? shift_up(uu[K - 1], u_last) : uu[k - 1];
                    du[k] = lm[k] * dt[k] * uu[k];
                    cp[k] = (dt[k] - lm[k] * dt[k]) * um1;
                } else {
                    du[k] = dt[k] * uu[k];
                }
                y[k] = Dd * uu[k];
                sum_dt += dt[k];
            }
            if constexpr (TRAP) u_last = readlane(uu[K - 1], 63);
        }
        // States entering the lanes that start a chunk: gathered in the wavefront's cells
        // (row 2 + chunk of the tile) and stored after the state loop -- a store inside the
        // loop would make every later load wait for it.
        static_assert(TILE == kCpt * kChunk, "chunks per tile");

        for (int n = 0; n < N; ++n, ++g) {
            // one compare of scalars each (an || of two compares would be carried through a
            // VGPR)
            const bool more = STAGE && (n + 1 < N || tile + TILE < L);  // a next state
            const bool mine = (g & 1) == par;  // HALVES: this state is staged by this half
            if (HALVES && mine) {
                // the rows of the state two after this one (wrapping into the next tiles)
                int n2 = n + 2, t2 = tile;
                while (n2 >= N) {  // at most twice (N >= 1)
                    n2 -= N;
                    t2 += TILE;
                }
                if (t2 < L) st.load(stid, rows(n2), t2, L);
            } else if (!HALVES && more) {  // the next state's rows
                st.load(stid, rows(n + 1 < N ? n + 1 : 0), n + 1 < N ? tile : tile + TILE, L);
            }
            const float An = cA[MSEL_IDX(n, kMaxN)];
            const float cn = cH[MSEL_IDX(n, kMaxN)];  // read early: used right after the scan
            float a[K], bb[K], bc[K];
            if constexpr (STAGE) Stage::read(stage[buf], 0, lane, bc);
            else load_k_cached<T, K, VEC>(Bb + static_cast<size_t>(MSEL_IDX(n, N)) * L, t0, L, bc);
            float bprev0 = 0.0f;  // TRAP: B_{n} of the step before the lane's first
            if constexpr (TRAP) {
                bprev0 = shift_up(bc[K - 1], readlane(B_last, n));
                B_last = writelane(readlane(bc[K - 1], 63), n, B_last);
            }
            float h = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                a[k] = exp2_hw(dt[k] * An);
                if constexpr (TRAP)
                    bb[k] = fmaf(a[k], cp[k] * (k == 0 ? bprev0 : bc[k - 1]), du[k] * bc[k]);
                else
                    bb[k] = du[k] * bc[k];
                h = k == 0 ? bb[0] : fmaf(a[k], h, bb[k]);  // the chain from a zero state
            }
            // without the stage the C rows' loads are issued here, where the B values are no
            // longer needed, and are in flight during the scan
            [[maybe_unused]] Raw<T, K> rcn;
            if constexpr (!STAGE)
                load_raw<T, K, VEC>(Cb + static_cast<size_t>(MSEL_IDX(n, N)) * L, t0, L, rcn);
            float P = exp2_hw(An * sum_dt);
            float S = h;
            scan_fwd_fused(P, S);
            const float Q = fmaf(P, cn, S);       // state after the lane's last step
            const float hin = shift_up(Q, cn);    // state entering the lane
            if (lane == 63) cH[MSEL_IDX(n, kMaxN)] = Q;
            if (lane % (kChunk / K) == 0)  // the first lane of a chunk
                cells[wave][MSEL_IDX(2 + lane / (kChunk / K), 2 + kCpt)][MSEL_IDX(n, kMaxN)] = hin;

            if constexpr (STAGE) Stage::read(stage[buf], 1, lane, bc);
            else unpack(rcn, bc);
            h = hin;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                h = fmaf(a[k], h, bb[k]);
                y[k] = fmaf(bc[k], h, y[k]);
            }
            if constexpr (STAGE) {
                if (more && (!HALVES || !mine)) st.store(stid, stage[buf ^ 1]);  // the next state
                __syncthreads();
                buf ^= 1;
            }
        }
        if constexpr (HAS_Z) {
            float zz[K];
            load_k_cached<T, K, VEC>(zr, t0, L, zz);
#pragma unroll
            for (int k = 0; k < K; ++k) y[k] *= zz[k] * sigmoid_f(zz[k]);
        }
        if (active) store_k<T, K, VEC, false>(out, t0, L, y);
        if (active && p.chunk_states != nullptr && lane < N) {
#pragma unroll
            for (int q = 0; q < kCpt; ++q) {
                const int cidx = tile / kChunk + q;
                if (cidx < p.nchunks)
                    p.chunk_states[MSEL_IDX((static_cast<size_t>(ch) * p.nchunks + cidx) * N + lane,
                                            BDN * p.nchunks)] = cells[wave][2 + q][lane];
            }
        }
    }
    if (active && p.final_state != nullptr && lane < N)
        p.final_state[MSEL_IDX(static_cast<size_t>(ch) * N + lane, BDN)] = cH[lane];
}

// Recurrent mode (page 3, recurrent mode; page 1 and 2: the state kept in a cache): one
// step per channel with the carried state, for decoding.  A 16-lane row per channel, lane n
// for state n (lanes n >= N idle), four channels per wavefront:
//   h_n = exp(Delta A_n) h0_n + Delta B_n u,  y = sum_n C_n h_n + D u,  out = y silu(z).
// The sum over states is a 16-lane DPP reduction.  final_state may be h0 itself (the state is
// updated in place): each lane reads its h0 before writing.
// TRAP adds the previous step's input, carried over the step: the trapezoidal rule above with
// u_{-1} = u_prev[b, d] and B_{-1} = B_prev[b, n].
template <typename T, bool HAS_Z, bool SOFTPLUS, bool TRAP>
__global__ __launch_bounds__(256) void scan_step_kernel(ScanParams p) {
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
    const int nc = n < N ? n : N - 1;
    const float u = Elem<T>::load1(static_cast<const T*>(p.u) + chc);
    const float x = Elem<T>::load1(static_cast<const T*>(p.delta) + chc) +
                    (p.bias ? p.bias[MSEL_IDX(d, p.D)] : 0.0f);
    const float dt = SOFTPLUS ? softplus_f(x) : x;
    // B and C are [batch, dstate, 1]
    const size_t bn = MSEL_IDX(static_cast<size_t>(b) * N + nc, static_cast<size_t>(p.B) * N);
    const float Bv = Elem<T>::load1(static_cast<const T*>(p.Bm) + bn);
    const float Cv = Elem<T>::load1(static_cast<const T*>(p.Cm) + bn);
    const float An = p.A[MSEL_IDX(static_cast<size_t>(d) * N + nc, static_cast<size_t>(p.D) * N)] * kLog2e;
    const size_t sidx = MSEL_IDX(static_cast<size_t>(chc) * N + nc, static_cast<size_t>(BD) * N);
    const float h0 = p.h0 ? p.h0[sidx] : 0.0f;
    const float a = exp2_hw(dt * An);
    float h;
    if constexpr (TRAP) {
        const float lm = Elem<T>::load1(static_cast<const T*>(p.lam) + chc);
        const float up = p.u_prev ? Elem<T>::load1(static_cast<const T*>(p.u_prev) + chc) : 0.0f;
        const float bp = p.B_prev ? Elem<T>::load1(static_cast<const T*>(p.B_prev) + bn) : 0.0f;
        h = fmaf(a, fmaf((dt - lm * dt) * up, bp, h0), lm * dt * u * Bv);
    } else {
        h = fmaf(a, h0, dt * Bv * u);
    }
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
        if (p.chunk_states != nullptr) p.chunk_states[sidx] = h0;  // one chunk: its entry state
        if (p.final_state != nullptr) p.final_state[sidx] = h;
    }
    if (in && n == 15) {
        float y = part + (p.Dv ? p.Dv[MSEL_IDX(d, p.D)] : 0.0f) * u;
        if constexpr (HAS_Z) {
            const float z = Elem<T>::load1(static_cast<const T*>(p.z) + chc);
            y *= z * sigmoid_f(z);
        }
        Elem<T>::store1(static_cast<T*>(p.out) + chc, y);
    }
}

namespace {

template <typename T, int K, bool VEC, bool HAS_Z, bool SP, bool TRAP>
hipError_t fwd_launch(const ScanParams& p, hipStream_t s) {
    // a workgroup per (batch row, W channels): its wavefronts share B and C
    constexpr int W = fwd_waves<T, TRAP>();
    const long long groups = static_cast<long long>(p.B) * ((p.D + W - 1) / W);
    hipLaunchKernelGGL((scan_fwd_kernel<T, K, VEC, HAS_Z, SP, TRAP>),
                       dim3(static_cast<unsigned>(groups)), dim3(64 * W), 0, s, p);
    return hipGetLastError();
}

template <typename T, int K, bool VEC, bool HAS_Z, bool SP>
hipError_t fwd_go(const ScanParams& p, hipStream_t s) {
    if (p.lam != nullptr) return fwd_launch<T, K, VEC, HAS_Z, SP, true>(p, s);
    return fwd_launch<T, K, VEC, HAS_Z, SP, false>(p, s);
}

template <typename T, int K>
hipError_t fwd_dispatch(const ScanParams& p, hipStream_t s) {
    const bool vec = (static_cast<size_t>(p.L) * sizeof(T)) % 16 == 0;
    const bool hz = p.z != nullptr;
    const bool sp = p.softplus != 0;
#define MSEL_FWD(V, Z, S) \
    if (vec == V && hz == Z && sp == S) return fwd_go<T, K, V, Z, S>(p, s);
    MSEL_FWD(true, true, true)
    MSEL_FWD(true, true, false)
    MSEL_FWD(true, false, true)
    MSEL_FWD(true, false, false)
    MSEL_FWD(false, true, true)
    MSEL_FWD(false, true, false)
    MSEL_FWD(false, false, true)
    MSEL_FWD(false, false, false)
#undef MSEL_FWD
    return hipErrorInvalidValue;
}

}  // namespace

template <typename T>
hipError_t step_dispatch(const ScanParams& p, hipStream_t s) {
    const long long threads = static_cast<long long>(p.B) * p.D * 16;
    dim3 grid(static_cast<unsigned>((threads + 255) / 256)), block(256);
    const bool hz = p.z != nullptr, sp = p.softplus != 0, tr = p.lam != nullptr;
#define MSEL_STEP(Z, S, R) \
    if (hz == Z && sp == S && tr == R) \
        hipLaunchKernelGGL((scan_step_kernel<T, Z, S, R>), grid, block, 0, s, p);
    MSEL_STEP(true, true, false)
    MSEL_STEP(true, false, false)
    MSEL_STEP(false, true, false)
    MSEL_STEP(false, false, false)
    MSEL_STEP(true, true, true)
    MSEL_STEP(true, false, true)
    MSEL_STEP(false, true, true)
    MSEL_STEP(false, false, true)
#undef MSEL_STEP
    return hipGetLastError();
}

hipError_t launch_scan_fwd(const ScanParams& p, bool bf16, hipStream_t stream) {
    if (p.L == 1) return bf16 ? step_dispatch<bf16_t>(p, stream) : step_dispatch<float>(p, stream);
    if (bf16) return fwd_dispatch<bf16_t, 16>(p, stream);
    return fwd_dispatch<float, 16>(p, stream);
}

// The checked build's test of its own checks: index `i` of a one-element array, which
// MSEL_IDX counts and redirects to element 0 when i != 0 (launched by the checked build only:
// the release build has no check and would store out of range).
__device__ float g_selftest_cell[1];

__global__ void bounds_selftest_kernel(int i) {
    if (threadIdx.x == 0) g_selftest_cell[MSEL_IDX(i, 1)] = 1.0f;
}

hipError_t launch_bounds_selftest(int i, hipStream_t stream) {
#ifdef MSEL_CHECKED
    hipLaunchKernelGGL(bounds_selftest_kernel, dim3(1), dim3(64), 0, stream, i);
    return hipGetLastError();
#else
    (void)i;
    (void)stream;
    return hipErrorNotSupported;
#endif
}

MSEL_BOUNDS_TAKER(take_bounds_fwd)

}  // namespace msel
