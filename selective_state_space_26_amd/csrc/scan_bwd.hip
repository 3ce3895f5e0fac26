// scan_bwd.hip -- backward selective scan with recomputation, for gfx950.
//
// Page 1 and page 4 (Appendix D, Memory paragraph): the intermediate states are not stored
// but recomputed in the backward pass from the inputs loaded from HBM.  Only one state per
// chunk of kChunk steps exists outside the chip.
//
// Gradients of a loss with respect to the inputs, given dout (a = exp(Delta A), y = C.h + D u
// before the gate, s = sigmoid(z)):
//   dy_t  = dout_t * z s                 dz_t = dout_t * y_t * s (1 + z (1 - s))
//   lam_t = C_t dy_t + a_{t+1} lam_{t+1} (adjoint of h_t, zero beyond the last step)
//   dC_t += dy_t h_t      dB_t += lam_t Delta_t u_t      (summed over channels)
//   g_t   = lam_t h_{t-1} a_t          dA += g_t Delta_t (summed over batch and time)
//   dDelta_t = sum_n (g_t A + lam_t B_t u_t)   du_t = sum_n lam_t Delta_t B_t + dy_t D
//   ddelta_t = dDelta_t * sigmoid(delta_t + bias) with the softplus, dbias += ddelta_t
//   dD += dy_t u_t       dh0 = a_0 lam_0
//
// Two plans (bwd_plan).  The chunk-parallel plan: three launches, all parallel over chunks:
//  1. summary: one wavefront per (batch, chunk, few channels).  For every state n it forms
//     the chunk's local end state from a zero start and the adjoint at the chunk's first step
//     from a zero adjoint beyond the chunk, in closed form from prefix sums of Delta (see the
//     kernel), plus sum(Delta) and Delta at the first step.  With the chunk states given only
//     the adjoint is formed, and chunk 0 is skipped unless dh0 is asked for.
//  2. link: one thread per (batch, channel, state) walks the chunks:
//       H_{c+1} = exp(A sum Delta_c) H_c + S_c                      (H_0 = h0)
//       G_{c-1} = exp(A sum Delta_c) G_c + exp(A Delta_first_c) Sr_c (G_last = 0)
//     H_c is the state entering chunk c, G_c = a lam at the first step after chunk c; the
//     walk ends with G = a_0 lam_0 = dh0.  (This is the chunk carry of page 4, Appendix D,
//     run once forward for the states and once backward for the adjoint.)  The same launch
//     zeroes the buffers that the main kernel adds into (dA, dB, dC, dD, dbias).
//  3. main: about one workgroup per compute unit, each on one (batch row, chunk) and a range
//     of channels; B and C of that chunk are staged in LDS once.  Each wavefront takes one
//     channel at a time: the states inside the chunk are rebuilt from H_c (lane chains and a
//     forward DPP scan), the adjoint from G_c (lane chains and the same scan in reversed lane
//     order), and every gradient term is formed in registers.  dB and dC, which sum over
//     channels, are accumulated over all the workgroup's channels in LDS and written to HBM
//     once per workgroup with fp32 global atomics.  LDS float atomics are avoided (they run at
//     a small fraction of the plain LDS rate on this chip): the wavefronts visit the states
//     in rotated order and hand each state's rows on in a ring, so a plain read-add-write
//     suffices.
// The fused plan (chunk states given, a few chunks): the main kernel alone, its workgroups
// each on (batch row, channel range) walking the chunks from the last to the first and
// carrying the adjoint between them itself (the link's backward walk, inside the kernel), then
// a reduce kernel that adds the workgroups' stored partial sums in a fixed order.
#include "msel_device.hpp"
#include "msel_kernels.hpp"

namespace msel {

constexpr int kSumWaves = 4;
constexpr int kMainWaves = 12;  // 3 per SIMD: the main kernel needs ~160 VGPRs
// The trapezoidal variant keeps ~50 more values per lane (the previous and next step's input
// terms and two more state sums): 2 wavefronts per SIMD.
constexpr int kTrapWaves = 8;
template <bool TRAP>
constexpr int main_waves() { return TRAP ? kTrapWaves : kMainWaves; }

struct BwdWork {
    float* H;       // [B*D*nch*N]: chunk-start states (may be the caller's chunk_states)
    float* G;       // [B*D*nch*N]: adjoint carry after each chunk
    float* sdt;     // [B*D*nch]: sum of Delta over the chunk
    float* dfirst;  // [B*D*nch]: Delta at the chunk's first step
    int want_fwd;   // the summary/link passes also build H
    int c0;         // first chunk summarised: chunk 0's adjoint summary feeds only dh0, so
                    // it is skipped (c0 = 1) when neither dh0 nor the states are built here
    FillList fill;  // the gradient kernel's reduction targets, zeroed by the link launch
    unsigned spin_limit;  // polls after which a ring wait gives up (ring_spin_limit())
    // The fused pass (bwd_plan): G is then the adjoint carry [B*D*N] of the chunk being
    // walked, and the sums over channels, batch rows and chunks go to partial sums that the
    // reduce kernel adds in a fixed order.
    float* part;    // [B][cgroups][nch][2][N][kChunk]: each workgroup's dB, dC rows per chunk
    float* dApart;  // [B][nch][D][N]
    float* dDpart;  // [B][nch][D]
    float* dbpart;  // [B][nch][D]
};

// Ring waits of this file's gradient kernel that gave up (see ring_spin_limit).
__device__ unsigned long long g_ring_timeouts_bwd;

std::atomic<unsigned> g_ring_spin_limit{kRingSpinDefault};

unsigned ring_spin_limit() { return g_ring_spin_limit.load(std::memory_order_relaxed); }

void set_ring_spin_limit(unsigned polls) {
    g_ring_spin_limit.store(polls != 0 ? polls : kRingSpinDefault, std::memory_order_relaxed);
}

hipError_t take_ring_timeouts_bwd(unsigned long long* count) {
    unsigned long long v = 0;
    const unsigned long long zero = 0;
    hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_ring_timeouts_bwd), sizeof(v), 0,
                                       hipMemcpyDeviceToHost);
    if (e == hipSuccess)
        e = hipMemcpyToSymbol(HIP_SYMBOL(g_ring_timeouts_bwd), &zero, sizeof(zero), 0,
                              hipMemcpyHostToDevice);
    *count = v;
    return e;
}

// Channels per wavefront in the summary: B and C rows are read (and converted) once per state
// and used for all of them.
template <bool FWD>
constexpr int sum_channels() { return FWD ? 2 : 4; }

// The summary needs only chunk totals, not the states at every step, so it uses the closed
// form of the recurrence instead of a scan: with E_t = sum of Delta over the chunk's steps
// 1..t (after its first step) and F'_t = sum of Delta over the steps after t,
//   adjoint at the chunk's first step, zero beyond the chunk:  sum_t exp(A E_t) C_t dy_t
//   end state from a zero start:                                sum_t exp(A F'_t) Delta_t u_t B_t
// (products of a = exp(Delta A) over a run of steps are exp(A * the run's sum of Delta)).  One
// prefix sum of Delta per channel replaces a scan per state, and every term is independent.
template <typename T, bool VEC, bool HAS_Z, bool SOFTPLUS, bool FWD>
__global__ __launch_bounds__(64 * kSumWaves) void bwd_summary_kernel(ScanParams p, GradParams g,
                                                                     BwdWork w) {
    constexpr int K = kChunk / 64;
    constexpr int R = sum_channels<FWD>();
    static_assert(FWD ? R == 2 : R == 4, "the reductions are done four at a time");
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nch = p.nchunks;
    const int dgroups = (p.D + R - 1) / R;
    const int nsum = nch - w.c0;  // chunks summarised
    const int idx = blockIdx.x * kSumWaves + wave;  // ((b * nsum) + c - c0) * dgroups + dg
    if (idx >= p.B * nsum * dgroups) return;
    const int dg = idx % dgroups;
    const int bc = idx / dgroups;
    const int c = w.c0 + bc % nsum;
    const int b = bc / nsum;
    const int L = p.L;
    const int N = p.N;
    const int t0 = c * kChunk + lane * K;
    const T* __restrict__ Bg =
        static_cast<const T*>(p.Bm) + static_cast<size_t>(MSEL_IDX(b, p.B)) * N * L;
    const T* __restrict__ Cg =
        static_cast<const T*>(p.Cm) + static_cast<size_t>(MSEL_IDX(b, p.B)) * N * L;
    [[maybe_unused]] const size_t BD = static_cast<size_t>(p.B) * p.D;

    // A slot past the last channel repeats channel D-1 exactly, so its results equal that
    // channel's and may be stored over them: every store is then unconditional, which keeps
    // the count of memory operations in flight known to the compiler (a conditional store
    // before a load makes the load's wait cover everything).
    int dch[R];
    float Av[R];       // lane n holds A[d, n] * log2(e)
    float E[R][K], dy[R][K];
    float Fs[FWD ? R : 1][K], du[FWD ? R : 1][K];
    // all input rows first, so that their loads are in flight together
    Raw<T, K> rd[R], rg[R], rz[HAS_Z ? R : 1], ru[FWD ? R : 1];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int d = dg * R + r;
        dch[r] = d < p.D ? d : p.D - 1;
        const size_t row = MSEL_IDX(static_cast<size_t>(b) * p.D + dch[r], BD) * L;
        load_raw<T, K, VEC>(static_cast<const T*>(p.delta) + row, t0, L, rd[r]);
        load_raw<T, K, VEC>(static_cast<const T*>(g.dout) + row, t0, L, rg[r]);
        if constexpr (HAS_Z) load_raw<T, K, VEC>(static_cast<const T*>(p.z) + row, t0, L, rz[r]);
        if constexpr (FWD) load_raw<T, K, VEC>(static_cast<const T*>(p.u) + row, t0, L, ru[r]);
        const float a_ = p.A[MSEL_IDX(static_cast<size_t>(dch[r]) * N + (lane < N ? lane : N - 1),
                                      static_cast<size_t>(p.D) * N)];
        Av[r] = (lane < N) ? a_ * kLog2e : 0.0f;
    }
    // E_t and F'_t are each summed from the steps they cover (the chunk's first step left
    // out of E; F'_t by a reversed lane scan), never as a difference of two sums: next to a
    // reset step's huge Delta such a difference would keep only a few bits of the remainder.
    const int rev_addr = (63 - lane) << 2;
    float tot[R], fst[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float bias = p.bias ? p.bias[MSEL_IDX(dch[r], p.D)] : 0.0f;
        float dd[K], gg[K], dt[K];
        unpack(rd[r], dd);
        unpack(rg[r], gg);
        float zz[HAS_Z ? K : 1], uu[FWD ? K : 1];
        if constexpr (HAS_Z) unpack(rz[r], zz);
        if constexpr (FWD) unpack(ru[r], uu);
        float run = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float x = dd[k] + bias;
            const float v = SOFTPLUS ? softplus_f(x) : x;
            dt[k] = (t0 + k < L) ? v : 0.0f;  // Delta = 0 past the end: identity step
            if constexpr (HAS_Z) dy[r][k] = gg[k] * zz[k] * sigmoid_f(zz[k]);
            else dy[r][k] = gg[k];
            if constexpr (FWD) du[r][k] = dt[k] * uu[k];
            run += (k == 0 && lane == 0) ? 0.0f : dt[k];  // the chunk's first step left out
            E[r][k] = run;  // inclusive within the lane for now
        }
        const float incl = wave_incl_sum(run);
        const float before = shift_up(incl, 0.0f);  // Delta summed over the earlier lanes
        fst[r] = readlane(dt[0], 0);
        tot[r] = readlane(incl, 63) + fst[r];
#pragma unroll
        for (int k = 0; k < K; ++k) E[r][k] += before;  // sum of Delta over steps 1..t
        if constexpr (FWD) {
            float suf = 0.0f;
#pragma unroll
            for (int k = K - 1; k >= 0; --k) {
                Fs[r][k] = suf;
                suf += dt[k];
            }
            const float after = wave_excl_suffix_sum(suf, rev_addr);
#pragma unroll
            for (int k = 0; k < K; ++k) Fs[r][k] += after;  // sum of Delta after t
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const size_t slot = MSEL_IDX((static_cast<size_t>(b) * p.D + dch[r]) * nch + c,
                                         BD * nch);
            w.sdt[slot] = tot[r];
            w.dfirst[slot] = fst[r];
        }
    }

    // results gathered per state (lane n = state n) and stored after the loop, so that the
    // loop's loads never wait behind stores
    float Gv[R] = {}, Hv[FWD ? R : 1] = {};
    Raw<T, K> Bn, Cn;
    if constexpr (FWD) load_raw<T, K, VEC>(Bg, t0, L, Bn);
    load_raw<T, K, VEC>(Cg, t0, L, Cn);
    for (int n = 0; n < N; ++n) {
        float bv[K], cv[K];
        if constexpr (FWD) unpack(Bn, bv);
        unpack(Cn, cv);
        {  // the next state's rows (the last state fetches its own again: no branch)
            const int nn = (n + 1 < N) ? n + 1 : n;
            if constexpr (FWD)
                load_raw<T, K, VEC>(Bg + static_cast<size_t>(MSEL_IDX(nn, N)) * L, t0, L, Bn);
            load_raw<T, K, VEC>(Cg + static_cast<size_t>(MSEL_IDX(nn, N)) * L, t0, L, Cn);
        }
        float acc[4];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float A2 = readlane(Av[r], n);
            float sg = 0.0f, sh = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                sg = fmaf(exp2_hw(A2 * E[r][k]), cv[k] * dy[r][k], sg);
                if constexpr (FWD) sh = fmaf(exp2_hw(A2 * Fs[r][k]), du[r][k] * bv[k], sh);
            }
            acc[r] = sg;
            if constexpr (FWD) acc[2 + r] = sh;
        }
        wave_sum4(acc[0], acc[1], acc[2], acc[3]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            Gv[r] = writelane(acc[r], n, Gv[r]);
            if constexpr (FWD) Hv[r] = writelane(acc[2 + r], n, Hv[r]);
        }
    }
    if (lane < N) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const size_t slot = MSEL_IDX(
                ((static_cast<size_t>(b) * p.D + dch[r]) * nch + c) * N + lane, BD * nch * N);
            w.G[slot] = Gv[r];
            if constexpr (FWD) w.H[slot] = Hv[r];
        }
    }
}

// One thread per (batch, channel, state) links the chunks; the launch also zeroes the gradient
// kernel's reduction targets (its grid may be wider than the links for that).
template <bool FWD>
__global__ __launch_bounds__(256) void bwd_link_kernel(ScanParams p, GradParams g, BwdWork w) {
    const size_t tid = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    zero_fill(w.fill, tid, static_cast<size_t>(gridDim.x) * blockDim.x);
    const int N = p.N;
    if (tid >= static_cast<size_t>(p.B) * p.D * N) return;
    const int ch = static_cast<int>(tid / N);  // < batch * dim, which fits an int
    const int n = static_cast<int>(tid - static_cast<size_t>(ch) * N);
    const int d = ch % p.D;
    const int nch = p.nchunks;
    [[maybe_unused]] const size_t BDN = static_cast<size_t>(p.B) * p.D * N;
    [[maybe_unused]] const size_t BDC = static_cast<size_t>(p.B) * p.D * nch;
    const float A2 = p.A[MSEL_IDX(static_cast<size_t>(d) * N + n, static_cast<size_t>(p.D) * N)] *
                     kLog2e;
    const size_t base = static_cast<size_t>(ch) * nch;
    if (FWD) {
        float H = p.h0 ? p.h0[MSEL_IDX(static_cast<size_t>(ch) * N + n, BDN)] : 0.0f;
        for (int c = 0; c < nch; ++c) {
            float* slot = w.H + MSEL_IDX((base + c) * N + n, BDC * N);
            const float S = *slot;
            *slot = H;
            H = fmaf(exp2_hw(A2 * w.sdt[MSEL_IDX(base + c, BDC)]), H, S);
        }
    }
    float G = 0.0f;
    for (int c = nch - 1; c >= w.c0; --c) {
        float* slot = w.G + MSEL_IDX((base + c) * N + n, BDC * N);
        const float Sr = *slot;
        *slot = G;
        G = fmaf(exp2_hw(A2 * w.sdt[MSEL_IDX(base + c, BDC)]), G,
                 exp2_hw(A2 * w.dfirst[MSEL_IDX(base + c, BDC)]) * Sr);
    }
    // the carry after chunk 0 (no summary of its own)
    if (w.c0 > 0) w.G[MSEL_IDX(base * N + n, BDC * N)] = G;
    if (g.dh0 != nullptr) g.dh0[MSEL_IDX(static_cast<size_t>(ch) * N + n, BDN)] = G;
}

// LDS layout of the main kernel:
//  * dB and dC accumulators [2 tensors][group][n][k][65] floats: the padded stride 65 keeps
//    both the per-lane updates (consecutive lanes) and the flush (consecutive time steps)
//    free of bank conflicts;
//  * B and C of the workgroup's (batch row, chunk) as fp32, [n][2 tensors][2][64 lanes][4]:
//    lane l's 8 steps are two 16-byte vectors, consecutive lanes adjacent (conflict-free), and
//    a state's four vectors per lane sit at constant offsets from one address;
//  * per-wave dA partials [wave][n][16]: sums over groups of four lanes, per state;
//  * kMaxN floats: B of every state at the step before the chunk (trapezoidal variant);
//  * (static) one int per (group, state): 1 + the global step of the last completed update
//    of that state's accumulator rows (see the ring protocol in the kernel).
constexpr int kAccKP = 65;
constexpr int kDaQuads = 16;
constexpr int kMaxRingFlags = 32;  // groups * N <= W + N - 1

__host__ __device__ constexpr int acc_groups(int N, int W) { return (W + N - 1) / N; }

__host__ __device__ constexpr size_t main_lds_bytes(int N, int W) {
    return (2 * static_cast<size_t>(acc_groups(N, W)) * N * (kChunk / 64) * kAccKP +
            2 * static_cast<size_t>(N) * kChunk + static_cast<size_t>(W) * N * kDaQuads +
            kMaxN) *
           sizeof(float);
}

// The largest need over 1 <= N <= kMaxN (it is not at kMaxN: fewer states can need more
// accumulator groups).
__host__ __device__ constexpr size_t main_lds_bytes_max(int W) {
    size_t m = 0;
    for (int n = 1; n <= kMaxN; ++n) m = main_lds_bytes(n, W) > m ? main_lds_bytes(n, W) : m;
    return m;
}
// static LDS of the main kernel besides the dynamic part: ring flags, per-wave cells and
// carries
__host__ __device__ constexpr size_t main_static_lds_bytes(int W) {
    return kMaxRingFlags * sizeof(int) + static_cast<size_t>(W) * kMaxN * (16 + 4);
}
static_assert(main_lds_bytes_max(kMainWaves) + main_static_lds_bytes(kMainWaves) <= 160 * 1024 &&
                  main_lds_bytes_max(kTrapWaves) + main_static_lds_bytes(kTrapWaves) <= 160 * 1024,
              "main kernel LDS exceeds a compute unit's 160 KB");
static_assert(kMainWaves + kMaxN - 1 <= kMaxRingFlags, "ring flags do not fit");

// TRAP: the exponential-trapezoidal rule, h_t = a_t (h_{t-1} + c_t B_{t-1}) + gam_t u_t B_t
// with gam_t = lam_t Delta_t and c_t = (1 - lam_t) Delta_t u_{t-1}.  The adjoint recurrence
// is unchanged; with at_t = a_{t+1} lam_{t+1} (the adjoint arriving from step t+1) the new
// terms are
//   dB_t += lam_t gam_t u_t + at_t c_{t+1}          g_t = lam_t a_t (h_{t-1} + c_t B_{t-1})
//   du_t  = gam_t sum_n lam B + (1 - lam_{t+1}) Delta_{t+1} sum_n at B + D dy_t
//   dlam_t = Delta_t (u_t sum_n lam B - u_{t-1} sum_n lam a B_{t-1})
//   dDelta_t = sum_n g_t A + lam_t u_t sum_n lam B + (1 - lam_t) u_{t-1} sum_n lam a B_{t-1}
// Step t-1's u and B come from the lane's registers, lane l-1, and for the chunk's first step
// from HBM (u) or the LDS row staged for it (B); step t+1's lam and Delta likewise from lane
// l+1 or the next chunk's first step.  The chunk states must be the trapezoidal forward's.
//
// FUSED (the plain rule with the chunk states given, see bwd_plan): one workgroup per (batch
// row, channel group) walks the chunks from the last to the first.  A wavefront keeps its
// channels in every chunk, so it carries each channel's adjoint from one chunk into the one
// before it itself (the value the scan leaves on the left of lane 0, through w.G), and no
// summary or link pass is needed; after chunk 0 that carry is dh0.  The sums over channels,
// batch rows and chunks are stored as partial sums, which the reduce kernel adds.
template <typename T, bool VEC, bool HAS_Z, bool SOFTPLUS, bool TRAP, bool FUSED>
__global__ __launch_bounds__(64 * main_waves<TRAP>()) void bwd_main_kernel(ScanParams p,
                                                                          GradParams g,
                                                                          BwdWork w,
                                                                          int per_wave) {
    static_assert(!(TRAP && FUSED), "the fused pass has the plain rule only");
    constexpr int K = kChunk / 64;
    constexpr int W = main_waves<TRAP>();
    constexpr int KP = kAccKP;
    // bf16 rows are small enough that the next channel's u and delta can be fetched during
    // the current channel's last step, next to this channel's z and dout (for dz)
    constexpr bool kEarlyUD = sizeof(T) == 2;
    extern __shared__ float acc[];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // one-dimensional grid over (batch row, chunk, channel group), channel groups fastest;
    // FUSED: over (batch row, channel group), starting at the last chunk
    const int cgroups = static_cast<int>(gridDim.x) / (FUSED ? p.B : p.B * p.nchunks);
    const int bc_ = static_cast<int>(blockIdx.x) / cgroups;
    const int cgrp = static_cast<int>(blockIdx.x) - bc_ * cgroups;
    const int b = FUSED ? bc_ : bc_ / p.nchunks;
    int c = FUSED ? p.nchunks - 1 : bc_ - b * p.nchunks;
    const int N = p.N;
    const int L = p.L;
    const int nch = p.nchunks;
    const int groups = acc_groups(N, W);
    const int tile = N * K * KP;             // floats per (tensor, group)
    float* accB = acc;
    float* accC = acc + groups * tile;
    float* BCs = acc + 2 * groups * tile;                   // B and C rows, by state
    float* dAs = BCs + 2 * N * kChunk + wave * N * kDaQuads;  // this wave's dA partials
    float* Bm1 = BCs + 2 * N * kChunk + W * N * kDaQuads;     // TRAP: B at step c*T - 1
    __shared__ int ring_flags[kMaxRingFlags];
    // Per wavefront and state, the channel's A, A log2(e), H_c and G_c (written once per
    // channel by lane n, read per step with one broadcast LDS read instead of v_readlane's),
    // and FUSED: the carry into the chunk before (written per step by the lane that has it).
    __shared__ f32x4 cells[W][kMaxN];
    __shared__ float gnext[FUSED ? W : 1][kMaxN];
    [[maybe_unused]] const size_t BD = static_cast<size_t>(p.B) * p.D;
    [[maybe_unused]] const size_t DN = static_cast<size_t>(p.D) * N;
    for (int i = tid; i < 2 * groups * tile; i += 64 * W) acc[i] = 0.0f;
    for (int i = tid; i < groups * N; i += 64 * W) ring_flags[MSEL_IDX(i, kMaxRingFlags)] = 0;
    int gstep = 0;  // the ring's global step (see below)
    for (;;) {  // FUSED: chunks nch-1 down to 0; otherwise the one chunk c
    const int t0 = c * kChunk + lane * K;
    const int rev_addr = (63 - lane) << 2;
    const f32x4* __restrict__ BC4 = reinterpret_cast<const f32x4*>(BCs);
    const T* __restrict__ gu = static_cast<const T*>(p.u);
    const T* __restrict__ gd = static_cast<const T*>(p.delta);
    const T* __restrict__ gg_ = static_cast<const T*>(g.dout);
    const T* __restrict__ gz = static_cast<const T*>(p.z);
    const T* __restrict__ gl = static_cast<const T*>(p.lam);
    auto chan_row = [&](int d) { return MSEL_IDX(static_cast<size_t>(b) * p.D + d, BD) * L; };

    // raw input rows of the channel about to start, fetched ahead of time: issued before the
    // chunk's B and C are staged, so that the two wait for L2 and HBM together
    Raw<T, K> ru, rd, rg, rz;
    Raw<T, K> rl;  // TRAP: lambda (unused otherwise)
    const int d_first = cgrp * per_wave * W + wave;
    if (d_first < p.D) {
        const size_t row = chan_row(d_first);
        load_raw<T, K, VEC>(gu + row, t0, L, ru);
        load_raw<T, K, VEC>(gd + row, t0, L, rd);
        if constexpr (TRAP) load_raw<T, K, VEC>(gl + row, t0, L, rl);
        load_raw<T, K, VEC>(gg_ + row, t0, L, rg);
        if constexpr (HAS_Z) load_raw<T, K, VEC>(gz + row, t0, L, rz);
    }

    {
        // B and C of this (batch row, chunk), read once per workgroup, zero past the end
        const T* __restrict__ Bg =
            static_cast<const T*>(p.Bm) + static_cast<size_t>(MSEL_IDX(b, p.B)) * N * L;
        const T* __restrict__ Cg =
            static_cast<const T*>(p.Cm) + static_cast<size_t>(MSEL_IDX(b, p.B)) * N * L;
        if constexpr (VEC) {
            // 16-byte vectors (a lane's K steps in bf16, half of them in fp32); a wavefront's
            // 64 vectors lie in one row, so the row is a scalar base.  Every load of the thread
            // is issued before its stores: one round trip to L2 per chunk, not one per element.
            constexpr int VW = Elem<T>::kPerVec;                      // elements per vector
            constexpr int RV = kChunk / VW;                           // vectors per row
            constexpr int kV = (kMaxN * RV + 64 * W - 1) / (64 * W);  // vectors per thread
            static_assert(RV % 64 == 0 && K % VW == 0 || VW % K == 0, "vector layout");
            f32x4* BCs4 = reinterpret_cast<f32x4*>(BCs);
            u32x4 rb[kV], rc[kV];
#pragma unroll
            for (int j = 0; j < kV; ++j) {
                const int v = tid + j * 64 * W;
                const int nn = __builtin_amdgcn_readfirstlane(v / RV);
                // no branch between the loads: a vector past the last state reads row 0 at
                // offset L, which is past the row's end, so it reads zeros (and is not stored)
                const bool in = nn < N;
                const int t = in ? c * kChunk + (v - nn * RV) * VW : L;
                const size_t row = static_cast<size_t>(in ? nn : 0) * L;
                rb[j] = load_vec<T, false>(Bg + row, t, L);
                rc[j] = load_vec<T, false>(Cg + row, t, L);
            }
#pragma unroll
            for (int j = 0; j < kV; ++j) {
                const int v = tid + j * 64 * W;
                const int nn = __builtin_amdgcn_readfirstlane(v / RV);
                if (nn >= N) break;
                const int tl = (v - nn * RV) * VW;  // the vector's first step in the chunk
                float fb[VW], fc[VW];
                unpack_vec<T, VW>(rb[j], 0, fb);
                unpack_vec<T, VW>(rc[j], 0, fc);
#pragma unroll
                for (int q = 0; q < VW / 4; ++q) {  // words (nn, B, (tl % K) / 4 + q) of lane tl / K
                    const int o =
                        MSEL_IDX((nn * 4 + (tl % K) / 4 + q) * 64 + tl / K, N * kChunk / 2 - 128);
                    BCs4[o] = f32x4{fb[4 * q], fb[4 * q + 1], fb[4 * q + 2], fb[4 * q + 3]};
                    BCs4[o + 128] = f32x4{fc[4 * q], fc[4 * q + 1], fc[4 * q + 2], fc[4 * q + 3]};
                }
            }
        } else {
            for (int i = tid; i < N * kChunk; i += 64 * W) {
                const int nn = i / kChunk;
                const int tl = i - nn * kChunk;
                const int t = c * kChunk + tl;
                float vb = 0.0f, vc = 0.0f;
                if (t < L) {
                    vb = Elem<T>::load1(Bg + static_cast<size_t>(nn) * L + t);
                    vc = Elem<T>::load1(Cg + static_cast<size_t>(nn) * L + t);
                }
                const int o = MSEL_IDX(((nn * 4 + (tl % K) / 4) * 64 + tl / K) * 4 + tl % 4,
                                       2 * N * kChunk - 512);
                BCs[o] = vb;
                BCs[o + 512] = vc;  // C: two words of 64 lanes further
            }
        }
        if constexpr (TRAP) {
            if (tid < N) {
                float v = 0.0f;
                if (c > 0)
                    v = Elem<T>::load1(Bg + static_cast<size_t>(tid) * L + c * kChunk - 1);
                else if (p.B_prev != nullptr)
                    v = Elem<T>::load1(static_cast<const T*>(p.B_prev) +
                                       MSEL_IDX(static_cast<size_t>(b) * N + tid,
                                                static_cast<size_t>(p.B) * N));
                Bm1[MSEL_IDX(tid, kMaxN)] = v;
            }
        }
    }
    __syncthreads();

    // Ring protocol for the shared accumulator rows.  The waves of a group take the states in
    // rotated order: at global step g (= channel round * N + step) wave `rot` updates state
    // (rot + g) mod N.  The previous update of that state was made kp steps earlier by wave
    // (rot + kp) mod N, kp = 1 unless rot is the group's last wave (then kp = N - rot, the
    // wrap to wave 0).  So each wave waits only for its ring successor's previous step, not
    // for the whole workgroup: a wave publishes the step it finished in its state's flag and
    // the next writer of that state spins on it.  Every wave runs every step (inactive ones
    // only publish), the chain ends at step 0, and all waves of the workgroup are resident,
    // so the waits always end.
    const int grp = wave / N;
    const int rot = wave - grp * N;
    const int Wg = (W - grp * N < N) ? W - grp * N : N;  // waves sharing this group's rows
    const int kp = (rot + 1 < Wg) ? 1 : N - rot;
    int* gflags = ring_flags + MSEL_IDX(grp * N, kMaxRingFlags);
    float* myB = accB + grp * tile;
    float* myC = accC + grp * tile;

    for (int r = 0; r < per_wave; ++r) {
        const int d = (cgrp * per_wave + r) * W + wave;
        const bool active = d < p.D;  // wave-uniform; inactive waves still run the protocol
        const bool next_active = (r + 1 < per_wave) && (d + W < p.D);
        const int dd_ = active ? d : 0;
        const size_t ch = MSEL_IDX(static_cast<size_t>(b) * p.D + dd_, BD);
        const size_t row = ch * L;
        const size_t row_next = chan_row(next_active ? d + W : 0);
        const float bias = p.bias ? p.bias[MSEL_IDX(dd_, p.D)] : 0.0f;
        const float Dd = p.Dv ? p.Dv[MSEL_IDX(dd_, p.D)] : 0.0f;
        // per-channel rows of A, H_c and G_c, one value per lane (lane n holds state n)
        const size_t hg = (ch * nch + c) * N;
        const float Av = (lane < N) ? p.A[MSEL_IDX(static_cast<size_t>(dd_) * N + lane, DN)] : 0.0f;
        const float Hv = (lane < N) ? w.H[MSEL_IDX(hg + lane, BD * nch * N)] : 0.0f;
        float Gv;
        if constexpr (FUSED)  // the carry of this channel from the chunk after (none after the last)
            Gv = c + 1 < nch ? load_lane(w.G + MSEL_IDX(ch, BD) * N, N, lane) : 0.0f;
        else
            Gv = (lane < N) ? w.G[MSEL_IDX(hg + lane, BD * nch * N)] : 0.0f;
        if (lane < N) cells[wave][lane] = f32x4{Av, Av * kLog2e, Hv, Gv};

        int n = rot;  // state of step 0

        float dt[K], dtu[K], dy[K], sB[K], sgA[K];
        // HAS_Z: y for dz, and dz's factor dout * silu'(z) = dout s (1 + z (1 - s)), formed
        // here beside dy with the same sigmoid s
        float y[HAS_Z ? K : 1], fz[HAS_Z ? K : 1];
        float sum_dt = 0.0f, dD_part = 0.0f;
        // TRAP: u, lambda, c_t, (1 - lam_{t+1}) Delta_{t+1}, c_{t+1}, u before the chunk, and
        // the sums of at B and of lam a B_{t-1}
        constexpr int KT = TRAP ? K : 1;
        float uT[KT], lm[KT], cp[KT], cnu[KT], cn[KT], sA[KT], sP[KT];
        float u_before = 0.0f;
        float cnu_after = 0.0f;  // (1 - lam) Delta at the next chunk's first step
        if constexpr (TRAP) {
            if (c > 0)
                u_before = Elem<T>::load1(gu + row + c * kChunk - 1);
            else if (p.u_prev != nullptr)
                u_before = Elem<T>::load1(static_cast<const T*>(p.u_prev) + ch);
            const int ta = (c + 1) * kChunk;
            if (ta < L) {
                const float x = Elem<T>::load1(gd + row + ta) + bias;
                const float da = SOFTPLUS ? softplus_f(x) : x;
                cnu_after = da - Elem<T>::load1(gl + row + ta) * da;
            }
        }
        {
            float uu[K], dd[K], go[K];
            unpack(ru, uu);
            unpack(rd, dd);
            unpack(rg, go);
            if constexpr (TRAP) unpack(rl, lm);
            float zz[HAS_Z ? K : 1];
            if constexpr (HAS_Z) unpack(rz, zz);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float x = dd[k] + bias;
                dt[k] = SOFTPLUS ? softplus_f(x) : x;
            }
            if ((c + 1) * kChunk > L) {  // Delta = 0 past the end: identity steps
#pragma unroll
                for (int k = 0; k < K; ++k) dt[k] = (t0 + k < L) ? dt[k] : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < K; ++k) {
                if constexpr (TRAP) {
                    uT[k] = uu[k];
                    dtu[k] = lm[k] * dt[k] * uu[k];
                    sA[k] = 0.0f;
                    sP[k] = 0.0f;
                } else {
                    dtu[k] = dt[k] * uu[k];
                }
                sum_dt += dt[k];
                if constexpr (HAS_Z) {
                    const float sg = sigmoid_f(zz[k]);
                    dy[k] = go[k] * zz[k] * sg;
                    fz[k] = go[k] * sg * fmaf(zz[k], 1.0f - sg, 1.0f);
                    y[k] = Dd * uu[k];
                } else {
                    dy[k] = go[k];
                }
                dD_part = fmaf(dy[k], uu[k], dD_part);
                sB[k] = 0.0f;
                sgA[k] = 0.0f;
            }
            if constexpr (TRAP) {
                const float um1 = shift_up(uu[K - 1], u_before);
#pragma unroll
                for (int k = 0; k < K; ++k)
                    cp[k] = (dt[k] - lm[k] * dt[k]) * (k == 0 ? um1 : uu[k - 1]);
                const float cnu_next = shift_down(dt[0] - lm[0] * dt[0], cnu_after);
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    cnu[k] = (k + 1 < K) ? dt[k + 1] - lm[k + 1] * dt[k + 1] : cnu_next;
                    cn[k] = cnu[k] * uu[k];
                }
            }
        }

        // One step: state nc of this channel.  `last` (the final state) also fetches inputs
        // for dz and the next channel, and finishes dz, which needs y summed over every state.
        auto step = [&](const bool last) __attribute__((always_inline)) {
            const int nc = n;
            const f32x4 cell = cells[wave][MSEL_IDX(nc, kMaxN)];  // A, A log2(e), H_c, G_c
            float bv[K], cv[K];
            {
                // state nc's vectors: B steps 0-3 and 4-7, then C's, 64 words apart
                const f32x4* bc = BC4 + MSEL_IDX(nc * 256 + lane, N * kChunk / 2 - 192);
                const f32x4 b0 = bc[0], b1 = bc[64], c0 = bc[128], c1 = bc[192];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    bv[q] = b0[q];
                    bv[4 + q] = b1[q];
                    cv[q] = c0[q];
                    cv[4 + q] = c1[q];
                }
            }
            if (!last) {
                n = (n + 1 == N) ? 0 : n + 1;
            } else {
                // no branches around these loads: for a channel that is not there they start
                // past the row's end (zeros, no memory access), so that the waits for them
                // count exactly the loads issued after them
                if constexpr (kEarlyUD) {
                    const int tn = next_active ? t0 : L;
                    load_raw<T, K, VEC>(gu + row_next, tn, L, ru);
                    load_raw<T, K, VEC>(gd + row_next, tn, L, rd);
                    if constexpr (TRAP) load_raw<T, K, VEC>(gl + row_next, tn, L, rl);
                }
            }
            // wait until the previous update of state nc (step gstep - kp) is complete
            const int need = gstep - kp + 1;
            if (need > 0) {
                unsigned polls = 0;
                while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(
                           gflags + MSEL_IDX(nc, kMaxRingFlags - grp * N), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP)) < need) {
                    if (++polls >= w.spin_limit) {  // give up: counted, never a hang
                        if (lane == 0)
                            __hip_atomic_fetch_add(&g_ring_timeouts_bwd, 1ull, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            asm volatile("" ::: "memory");
            if (active) {
                // this step's accumulator slots: each tensor's reads are issued together,
                // ahead of their use, and written back as soon as its pass is done
                // rows k = 0 .. K-1 of this step are sBn[k * KP] (the base's extent leaves
                // room for them and the 64 lanes)
                float* sBn = myB + MSEL_IDX(nc * K * KP, tile - (K - 1) * KP - 63) + lane;
                float* sCn = myC + MSEL_IDX(nc * K * KP, tile - (K - 1) * KP - 63) + lane;
                float oc[K];
#pragma unroll
                for (int k = 0; k < K; ++k) oc[k] = sCn[k * KP];
                const float An = cell[0];
                const float An2 = cell[1];
                const float Hn = cell[2];
                const float Gn = cell[3];
                // lane-local chains: states from a zero start, adjoint from a zero end
                float a[K], bb[K], cd[K];
                float bp0 = 0.0f;  // TRAP: B of state nc at the step before the lane's first
                if constexpr (TRAP) bp0 = shift_up(bv[K - 1], Bm1[nc]);
                float h = 0.0f;
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    a[k] = exp2_hw(dt[k] * An2);
                    if constexpr (TRAP)
                        bb[k] = fmaf(a[k], cp[k] * (k == 0 ? bp0 : bv[k - 1]), dtu[k] * bv[k]);
                    else
                        bb[k] = dtu[k] * bv[k];
                    h = k == 0 ? bb[0] : fmaf(a[k], h, bb[k]);  // the chain from a zero state
                    cd[k] = cv[k] * dy[k];
                }
                // the lane's adjoint chain from a zero input on its right
                float rr = cd[K - 1];
#pragma unroll
                for (int k = K - 2; k >= 0; --k) rr = fmaf(a[k + 1], rr, cd[k]);
                // Lane maps.  States: x -> P x + S with P = a_{K-1} ... a_0.  Adjoints: from the
                // one arriving on the lane's right (carried into its last step) to the one
                // leaving on its left (carried into the previous lane's last step),
                // x -> P x + a_0 rr, the same P.  The adjoint maps are scanned forward in
                // reversed lane order, next to the states' scan.
                float P = exp2_hw(An2 * sum_dt), S = h;
                float Pr = rev_lanes(P, rev_addr), Sr = rev_lanes(a[0] * rr, rev_addr);
                scan_fwd2_fused(P, S, Pr, Sr);
                // state entering the lane (from H_c)
                const float hin = shift_up(fmaf(P, Hn, S), Hn);
                // reversed lane 63 - l now maps G_c to the adjoint leaving lane l on its left;
                // lane l receives lane l + 1's (G_c for lane 63), carried into its last step
                const float Gl = fmaf(Pr, Gn, Sr);
                if constexpr (FUSED)  // reversed lane 63: the adjoint leaving lane 0
                    if (lane == 63) gnext[0][MSEL_IDX(wave * kMaxN + nc, W * kMaxN)] = Gl;
                float lam = rev_lanes(shift_up(Gl, Gn), rev_addr);
                float hs[K];
                h = hin;
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    h = fmaf(a[k], h, bb[k]);
                    hs[k] = h;
                    if constexpr (HAS_Z) y[k] = fmaf(cv[k], h, y[k]);
                    oc[k] = fmaf(dy[k], h, oc[k]);
                }
                float ob[K];
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    sCn[k * KP] = oc[k];
                    ob[k] = sBn[k * KP];
                }
                if constexpr (HAS_Z) {
                    if (last) {  // y is complete: dz = dout * y * silu'(z)
                        float o[K];
#pragma unroll
                        for (int k = 0; k < K; ++k) o[k] = fz[k] * y[k];
                        store_k<T, K, VEC>(static_cast<T*>(g.dz) + row, t0, L, o);
                    }
                }
                float dA_part = 0.0f;
                float first_lac = 0.0f;  // TRAP: lam_0 a_0 c_0 of the lane's first step
#pragma unroll
                for (int k = K - 1; k >= 0; --k) {
                    if constexpr (TRAP) {
                        const float at = (k == K - 1) ? lam : a[k + 1] * lam;
                        lam = at + cd[k];
                        const float bpk = (k == 0) ? bp0 : bv[k - 1];
                        const float hprev = fmaf(cp[k], bpk, (k == 0) ? hin : hs[k - 1]);
                        const float la = lam * a[k];
                        const float gk = la * hprev;
                        dA_part = fmaf(gk, dt[k], dA_part);
                        sgA[k] = fmaf(gk, An, sgA[k]);
                        sB[k] = fmaf(lam, bv[k], sB[k]);
                        sA[k] = fmaf(at, bv[k], sA[k]);
                        sP[k] = fmaf(la, bpk, sP[k]);
                        ob[k] = fmaf(lam, dtu[k], fmaf(at, cn[k], ob[k]));
                        if (k == 0) first_lac = la * cp[0];
                    } else {
                        lam = (k == K - 1) ? lam + cd[k] : fmaf(a[k + 1], lam, cd[k]);
                        const float hprev = (k == 0) ? hin : hs[k - 1];
                        const float gk = lam * hprev * a[k];
                        dA_part = fmaf(gk, dt[k], dA_part);
                        sgA[k] = fmaf(gk, An, sgA[k]);
                        sB[k] = fmaf(lam, bv[k], sB[k]);
                        ob[k] = fmaf(lam, dtu[k], ob[k]);
                    }
                }
#pragma unroll
                for (int k = 0; k < K; ++k) sBn[k * KP] = ob[k];
                // TRAP: dB_prev[b, n] sums lam_0 a_0 c_0 of the sequence's first step over
                // channels (the B_prev term of h_0)
                if constexpr (TRAP) {
                    if (c == 0 && lane == 0 && g.dB_prev != nullptr)
                        unsafeAtomicAdd(g.dB_prev + MSEL_IDX(static_cast<size_t>(b) * N + nc,
                                                             static_cast<size_t>(p.B) * N),
                                        first_lac);
                }
                const float dq = quad_sum(dA_part);
                if ((lane & 3) == 0) dAs[MSEL_IDX(nc * kDaQuads + (lane >> 2), N * kDaQuads)] = dq;
            }
            // publish: this step's LDS writes are complete
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __hip_atomic_store(gflags + MSEL_IDX(nc, kMaxRingFlags - grp * N), gstep + 1,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            ++gstep;
        };

        for (int j = 0; j + 1 < N; ++j) step(false);
        step(true);

        // this channel's delta (for the softplus derivative) and u again, for du and ddelta
        // (its rows, still in L2: one load costs fewer instructions than keeping them), issued
        // before the next channel's loads so that waiting for them does not wait for those
        if constexpr (FUSED) {  // the carry into the chunk before; after chunk 0 it is dh0
            if (active) {
                const float Gnext =
                    lane < N ? gnext[0][MSEL_IDX(wave * kMaxN + lane, W * kMaxN)] : 0.0f;
                if (c > 0)
                    store_lane(w.G + MSEL_IDX(ch, BD) * N, N, lane, Gnext);
                else if (g.dh0 != nullptr)
                    store_lane(g.dh0 + MSEL_IDX(ch, BD) * N, N, lane, Gnext);
            }
        }
        // (as in the last step, no branches around the loads below)
        [[maybe_unused]] Raw<T, K> rxs, ruu;
        if constexpr (SOFTPLUS) load_raw<T, K, VEC>(gd + row, active ? t0 : L, L, rxs);
        if constexpr (!TRAP) load_raw<T, K, VEC>(gu + row, active ? t0 : L, L, ruu);
        asm volatile("" ::: "memory");  // keep them ahead of the loads below
        // the rest of the next channel's inputs, in flight while this one is finished
        {
            const int tn = next_active ? t0 : L;
            if constexpr (!kEarlyUD) {
                load_raw<T, K, VEC>(gu + row_next, tn, L, ru);
                load_raw<T, K, VEC>(gd + row_next, tn, L, rd);
                if constexpr (TRAP) load_raw<T, K, VEC>(gl + row_next, tn, L, rl);
            }
            load_raw<T, K, VEC>(gg_ + row_next, tn, L, rg);
            if constexpr (HAS_Z) load_raw<T, K, VEC>(gz + row_next, tn, L, rz);
        }
        if (!active) continue;

        // du and ddelta.  With the softplus, ddelta = dDelta * sigmoid(delta + bias), formed
        // from delta + bias and Delta (softplus_grad_f).
        float o1[K], o2[K];
        float db_part = 0.0f;
        float xs[SOFTPLUS ? K : 1];  // delta + bias
        if constexpr (SOFTPLUS) {
            unpack(rxs, xs);
#pragma unroll
            for (int k = 0; k < K; ++k) xs[k] += bias;
        }
        if constexpr (TRAP) {
            float o3[K];
            const float um1_0 = shift_up(uT[K - 1], u_before);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float um1 = (k == 0) ? um1_0 : uT[k - 1];
                const float dsp = SOFTPLUS ? softplus_grad_f(xs[k], dt[k]) : 1.0f;
                o1[k] = fmaf(sB[k], lm[k] * dt[k], fmaf(sA[k], cnu[k], dy[k] * Dd));     // du
                const float dD_ = fmaf(sP[k], um1 - lm[k] * um1, fmaf(sB[k], lm[k] * uT[k], sgA[k]));
                o2[k] = dD_ * dsp;                                                       // ddelta
                o3[k] = dt[k] * fmaf(uT[k], sB[k], -um1 * sP[k]);                         // dlam
            }
            store_k<T, K, VEC>(static_cast<T*>(g.dlam) + row, t0, L, o3);
            // the u_prev term of h_0: (1 - lam_0) Delta_0 sum_n lam_0 a_0 B_prev
            if (c == 0 && lane == 0 && g.du_prev != nullptr)
                g.du_prev[ch] = (dt[0] - lm[0] * dt[0]) * sP[0];
        } else {
            float uu[K];
            unpack(ruu, uu);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float dsp = SOFTPLUS ? softplus_grad_f(xs[k], dt[k]) : 1.0f;
                o1[k] = fmaf(sB[k], dt[k], dy[k] * Dd);            // du
                o2[k] = fmaf(sB[k], uu[k], sgA[k]) * dsp;         // ddelta
            }
        }
        // dbias sums the chunk's ddelta; steps past the end are masked only in a chunk that
        // reaches past it
        if ((c + 1) * kChunk > L) {
#pragma unroll
            for (int k = 0; k < K; ++k) db_part += (t0 + k < L) ? o2[k] : 0.0f;
        } else {
#pragma unroll
            for (int k = 0; k < K; ++k) db_part += o2[k];
        }
        store_k<T, K, VEC>(static_cast<T*>(g.du) + row, t0, L, o1);
        store_k<T, K, VEC>(static_cast<T*>(g.ddelta) + row, t0, L, o2);
        // dA[d, n]: lane n sums the 16 quad partials of state n (the wave's own rows: same-wave
        // LDS order, no barrier needed)
        float sa = 0.0f;
        if (lane < N) {
            const f32x4* src =
                reinterpret_cast<const f32x4*>(dAs + MSEL_IDX(lane * kDaQuads, N * kDaQuads));
#pragma unroll
            for (int q = 0; q < kDaQuads / 4; ++q) {
                const f32x4 v = src[q];
                sa += (v[0] + v[1]) + (v[2] + v[3]);
            }
        }
        const float sD = wave_sum_fused(dD_part);
        const float sb = wave_sum_fused(db_part);
        if constexpr (FUSED) {  // this (batch row, chunk, channel)'s share, stored
            const size_t pc = MSEL_IDX((static_cast<size_t>(b) * nch + c) * p.D + d, BD * nch);
            if (g.dA != nullptr) store_lane(w.dApart + pc * N, N, lane, sa);  // lanes n < N
            if (g.dD != nullptr && lane == 62) w.dDpart[pc] = sD;
            if (g.dbias != nullptr && lane == 63) w.dbpart[pc] = sb;
            continue;
        }
        // one vector atomic per channel: lane n < N adds dA[d, n], lane 62 dD[d], 63 dbias[d]
        float* dst = nullptr;
        float val = 0.0f;
        if (lane < N) {
            dst = g.dA ? g.dA + MSEL_IDX(static_cast<size_t>(d) * N + lane, DN) : nullptr;
            val = sa;
        } else if (lane == 62) {
            dst = g.dD ? g.dD + MSEL_IDX(d, p.D) : nullptr;
            val = sD;
        } else if (lane == 63) {
            dst = g.dbias ? g.dbias + MSEL_IDX(d, p.D) : nullptr;
            val = sb;
        }
        if (dst != nullptr) unsafeAtomicAdd(dst, val);
    }

    __syncthreads();
    if constexpr (FUSED) {
        // this chunk's rows of the workgroup's dB and dC sums, stored whole (past the end of
        // the sequence too: the reduce kernel reads only steps < L); the accumulators are
        // zeroed for the chunk before.  (Plain stores: with non-temporal ones the sums leave
        // the last-level cache and the reduce kernel reads them from HBM, 4 us slower.)
        float* dst = w.part + MSEL_IDX(((static_cast<size_t>(b) * cgroups + cgrp) * nch + c) *
                                           2 * N * kChunk,
                                       static_cast<size_t>(p.B) * cgroups * nch * 2 * N * kChunk);
        for (int i = tid; i < N * kChunk; i += 64 * W) {
            const int nn = i / kChunk;
            const int tt = i - nn * kChunk;
            const int slot = (nn * K + tt % K) * KP + tt / K;
            float vb = 0.0f, vc = 0.0f;
            for (int q = 0; q < groups; ++q) {
                const int o = MSEL_IDX(q * tile + slot, groups * tile);
                vb += accB[o];
                vc += accC[o];
                accB[o] = 0.0f;
                accC[o] = 0.0f;
            }
            dst[i] = vb;
            dst[N * kChunk + i] = vc;
        }
        if (c == 0) break;
        --c;
        continue;  // the next chunk's staging follows; its barrier orders the zeroing
    }
    for (int i = tid; i < N * kChunk; i += 64 * W) {
        const int nn = i / kChunk;
        const int tt = i - nn * kChunk;
        const int t = c * kChunk + tt;
        if (t >= L) continue;
        const int slot = (nn * K + tt % K) * KP + tt / K;
        float vb = 0.0f, vc = 0.0f;
        for (int q = 0; q < groups; ++q) {
            vb += accB[MSEL_IDX(q * tile + slot, groups * tile)];
            vc += accC[MSEL_IDX(q * tile + slot, groups * tile)];
        }
        const size_t o =
            MSEL_IDX((static_cast<size_t>(b) * N + nn) * L + t, static_cast<size_t>(p.B) * N * L);
        if (g.dB != nullptr) unsafeAtomicAdd(g.dB + o, vb);
        if (g.dC != nullptr) unsafeAtomicAdd(g.dC + o, vc);
    }
    break;
    }  // chunks
}

// Zeroes up to kFillSlots buffers in one launch (for reductions with no launch of their own
// before them to do it, such as the convolution backward's).
__global__ void fill_zero_kernel(FillList f) {
    zero_fill(f, static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x,
              static_cast<size_t>(gridDim.x) * blockDim.x);
}

hipError_t launch_fill_zero(const FillList& f, hipStream_t stream) {
    const unsigned blocks = fill_blocks(f);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, stream, f);
    return hipGetLastError();
}

// The fused pass's reductions, each summed in a fixed order (so the fused backward is
// deterministic): dB and dC over the channel groups, dA, dD and dbias over batch rows and
// chunks.  Thread i < B*N*L: element i of dB and dC; the next D*N: dA; the next D: dD, dbias.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(ScanParams p, GradParams g, BwdWork w,
                                                         int cgroups) {
    const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int N = p.N, L = p.L, nch = p.nchunks;
    const size_t BNL = static_cast<size_t>(p.B) * N * L;
    const size_t DN = static_cast<size_t>(p.D) * N;
    const size_t BC = static_cast<size_t>(p.B) * nch;  // (batch row, chunk) partials
    if (i < BNL) {
        const size_t bn = i / L;
        const int t = static_cast<int>(i - bn * L);
        const int b = static_cast<int>(bn / N);
        const int n = static_cast<int>(bn - static_cast<size_t>(b) * N);
        const int c = t / kChunk;
        const size_t rows = static_cast<size_t>(nch) * 2 * N * kChunk;  // per channel group
        const size_t o = static_cast<size_t>(b) * cgroups * rows +
                         (static_cast<size_t>(c) * 2 * N + n) * kChunk + (t - c * kChunk);
        // eight groups' values loaded together, then added in group order
        const float* src = w.part + o;
        const size_t cw = static_cast<size_t>(N) * kChunk;  // from a group's dB rows to its dC
        float sb = 0.0f, sc = 0.0f;
        for (int j0 = 0; j0 < cgroups; j0 += 8) {
            float vb[8], vc[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const size_t at = static_cast<size_t>(j0 + q) * rows;
                const bool in = j0 + q < cgroups;
                vb[q] = in ? src[MSEL_IDX(at, BC * cgroups * 2 * N * kChunk - o)] : 0.0f;
                vc[q] = in ? src[MSEL_IDX(at + cw, BC * cgroups * 2 * N * kChunk - o)] : 0.0f;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                sb += vb[q];
                sc += vc[q];
            }
        }
        if (g.dB != nullptr) g.dB[i] = sb;
        if (g.dC != nullptr) g.dC[i] = sc;
        return;
    }
    size_t k = i - BNL;
    // the other sums: over (batch row, chunk) partials, eight loaded together and added in order
    auto sum_bc = [&](const float* part, size_t stride, size_t k_) {
        float acc = 0.0f;
        for (size_t j0 = 0; j0 < BC; j0 += 8) {
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                v[q] = j0 + q < BC ? part[MSEL_IDX((j0 + q) * stride + k_, BC * stride)] : 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) acc += v[q];
        }
        return acc;
    };
    if (k < DN) {
        if (g.dA != nullptr) g.dA[k] = sum_bc(w.dApart, DN, k);
        return;
    }
    k -= DN;
    if (k < static_cast<size_t>(p.D)) {
        if (g.dD != nullptr) g.dD[k] = sum_bc(w.dDpart, p.D, k);
        if (g.dbias != nullptr) g.dbias[k] = sum_bc(w.dbpart, p.D, k);
    }
}

std::atomic<int> g_bwd_fused_mode{0};

int bwd_fused_mode() { return g_bwd_fused_mode.load(std::memory_order_relaxed); }

void set_bwd_fused_mode(int mode) {
    g_bwd_fused_mode.store(mode > 0 ? 1 : (mode < 0 ? -1 : 0), std::memory_order_relaxed);
}

BwdPlan bwd_plan(int B, int D, int N, int L, bool need_states, size_t cap) {
    const size_t nch = (static_cast<size_t>(L) + kChunk - 1) / kChunk;
    const size_t states = static_cast<size_t>(B) * D * nch * N * sizeof(float);
    const size_t per_chunk = static_cast<size_t>(B) * D * nch * sizeof(float);
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    BwdPlan plan{};
    plan.bytes = (need_states ? up(states) : 0) + up(states) + 2 * up(per_chunk);
    const int mode = bwd_fused_mode();
    if (need_states || mode < 0 || N > kMaxN) return plan;
    // about kFusedWorkgroups workgroups of kMainWaves channels at a time; a pure function of
    // the sizes (the workspace size must not depend on the device)
    constexpr int W = kMainWaves;
    long long cg = (kFusedWorkgroups + B - 1) / B;
    const long long cg_max = (static_cast<long long>(D) + W - 1) / W;
    if (cg > cg_max) cg = cg_max;
    const long long per = (static_cast<long long>(D) + cg * W - 1) / (cg * W);
    cg = (static_cast<long long>(D) + per * W - 1) / (per * W);
    const size_t fused = up(static_cast<size_t>(B) * D * N * sizeof(float)) +          // carry
                         up(static_cast<size_t>(B) * cg * nch * 2 * N * kChunk * 4) +  // dB, dC
                         up(static_cast<size_t>(B) * nch * D * N * sizeof(float)) +    // dA
                         2 * up(per_chunk);                                             // dD, dbias
    const size_t bytes = fused > plan.bytes ? fused : plan.bytes;
    if (bytes > cap) return plan;
    // automatically: a few chunks (the partial sums grow with the sequence, the summary the
    // fused pass saves does not) and enough workgroups to fill most of the chip
    if (mode == 0 && (nch > kFusedMaxChunks || B * cg < kFusedWorkgroups / 2)) return plan;
    plan.fused = true;
    plan.cgroups = static_cast<int>(cg);
    plan.per_wave = static_cast<int>(per);
    plan.bytes = bytes;
    return plan;
}

size_t bwd_workspace_bytes(int B, int D, int N, int L, bool need_states, size_t cap) {
    return bwd_plan(B, D, N, L, need_states, cap).bytes;
}

namespace {

// Channels per wavefront in the main kernel: about one workgroup per compute unit, so that
// each workgroup walks many channels of one (batch row, chunk) and flushes its dB/dC sums once.
int main_per_wave(const ScanParams& p, int waves) {
    const int cus = device_compute_units();
    const long long slots = static_cast<long long>(p.B) * p.nchunks;
    const long long target = cus;
    long long per = (static_cast<long long>(p.D) * slots + target * waves - 1) /
                    (target * waves);
    const long long max_per = (p.D + waves - 1) / waves;
    if (per < 1) per = 1;
    if (per > max_per) per = max_per;
    return static_cast<int>(per);
}

struct Timing {
    hipEvent_t begin, end;
};

// The fused plan: the gradient kernel over (batch row, channel group), then the reduce kernel.
template <typename T, bool VEC, bool HAS_Z, bool SP>
hipError_t bwd_fused_go(const ScanParams& p, const GradParams& g, const BwdWork& w,
                        const BwdPlan& plan, hipStream_t s, Timing tm) {
    constexpr int W = main_waves<false>();
    hipError_t e = allow_dynamic_lds<&bwd_main_kernel<T, VEC, HAS_Z, SP, false, true>>(
        static_cast<int>(main_lds_bytes_max(W)));
    if (e != hipSuccess) return e;
    const long long mblocks = static_cast<long long>(plan.cgroups) * p.B;
    if (mblocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (tm.begin != nullptr && (e = hipEventRecord(tm.begin, s)) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_main_kernel<T, VEC, HAS_Z, SP, false, true>),
                       dim3(static_cast<unsigned>(mblocks)), dim3(64 * W), main_lds_bytes(p.N, W),
                       s, p, g, w, plan.per_wave);
    e = hipGetLastError();
    if (e == hipSuccess && tm.end != nullptr) e = hipEventRecord(tm.end, s);
    if (e != hipSuccess) return e;
    const size_t threads = static_cast<size_t>(p.B) * p.N * p.L +
                           static_cast<size_t>(p.D) * p.N + static_cast<size_t>(p.D);
    const size_t rblocks = (threads + 255) / 256;
    if (rblocks > 0x7fffffffULL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3(static_cast<unsigned>(rblocks)), dim3(256), 0, s,
                       p, g, w, plan.cgroups);
    return hipGetLastError();
}

template <typename T, bool VEC, bool HAS_Z, bool SP, bool TRAP>
hipError_t bwd_go(const ScanParams& p, const GradParams& g, const BwdWork& w,
                  const BwdPlan& plan, hipStream_t s, Timing tm) {
    if constexpr (!TRAP) {
        if (plan.fused) return bwd_fused_go<T, VEC, HAS_Z, SP>(p, g, w, plan, s, tm);
    }
    constexpr int W = main_waves<TRAP>();
    const int per_sum = w.want_fwd ? sum_channels<true>() : sum_channels<false>();
    const int sum_waves = p.B * (p.nchunks - w.c0) * ((p.D + per_sum - 1) / per_sum);
    dim3 sgrid((sum_waves + kSumWaves - 1) / kSumWaves), sblock(64 * kSumWaves);
    if (w.want_fwd)
        hipLaunchKernelGGL((bwd_summary_kernel<T, VEC, HAS_Z, SP, true>), sgrid, sblock, 0, s, p,
                           g, w);
    else if (sum_waves > 0)  // none with a single chunk and no dh0
        hipLaunchKernelGGL((bwd_summary_kernel<T, VEC, HAS_Z, SP, false>), sgrid, sblock, 0, s, p,
                           g, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long links = static_cast<long long>(p.B) * p.D * p.N;  // may exceed an int
    const unsigned fb = fill_blocks(w.fill);
    dim3 lgrid(std::max(static_cast<unsigned>((links + 255) / 256), fb)), lblock(256);
    if (w.want_fwd)
        hipLaunchKernelGGL(bwd_link_kernel<true>, lgrid, lblock, 0, s, p, g, w);
    else
        hipLaunchKernelGGL(bwd_link_kernel<false>, lgrid, lblock, 0, s, p, g, w);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int per_wave = main_per_wave(p, W);
    const int cgroups = (p.D + per_wave * W - 1) / (per_wave * W);
    const size_t lds = main_lds_bytes(p.N, W);
    // the LDS exceeds the 64 KB default; allow the largest need over N <= kMaxN
    e = allow_dynamic_lds<&bwd_main_kernel<T, VEC, HAS_Z, SP, TRAP, false>>(
        static_cast<int>(main_lds_bytes_max(W)));
    if (e != hipSuccess) return e;
    const long long mblocks = static_cast<long long>(cgroups) * p.nchunks * p.B;
    if (mblocks > 0x7fffffffLL) return hipErrorInvalidValue;
    dim3 mgrid(static_cast<unsigned>(mblocks)), mblock(64 * W);
    if (tm.begin != nullptr && (e = hipEventRecord(tm.begin, s)) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_main_kernel<T, VEC, HAS_Z, SP, TRAP, false>), mgrid, mblock, lds, s,
                       p, g, w, per_wave);
    e = hipGetLastError();
    if (e == hipSuccess && tm.end != nullptr) e = hipEventRecord(tm.end, s);
    return e;
}

template <typename T>
hipError_t bwd_dispatch(const ScanParams& p, const GradParams& g, const BwdWork& w,
                        const BwdPlan& plan, hipStream_t s, Timing tm) {
    const bool vec = (static_cast<size_t>(p.L) * sizeof(T)) % 16 == 0;
    const bool hz = p.z != nullptr;
    const bool sp = p.softplus != 0;
    if (p.lam != nullptr) {  // the trapezoidal variant (chunk states given by its forward)
#define MSEL_BWD_T(V, Z, S) \
        if (vec == V && hz == Z && sp == S) return bwd_go<T, V, Z, S, true>(p, g, w, plan, s, tm);
        MSEL_BWD_T(true, true, true)
        MSEL_BWD_T(true, true, false)
        MSEL_BWD_T(true, false, true)
        MSEL_BWD_T(true, false, false)
        MSEL_BWD_T(false, true, true)
        MSEL_BWD_T(false, true, false)
        MSEL_BWD_T(false, false, true)
        MSEL_BWD_T(false, false, false)
#undef MSEL_BWD_T
        return hipErrorInvalidValue;
    }
#define MSEL_BWD(V, Z, S) \
    if (vec == V && hz == Z && sp == S) return bwd_go<T, V, Z, S, false>(p, g, w, plan, s, tm);
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
                           void* workspace, size_t workspace_bytes, bool bf16,
                           const FillList& fill, hipStream_t stream, hipEvent_t ev_begin,
                           hipEvent_t ev_end) {
    if (p.N > kMaxN) return hipErrorInvalidValue;
    const size_t nch = static_cast<size_t>(p.nchunks);
    const size_t states = static_cast<size_t>(p.B) * p.D * nch * p.N * sizeof(float);
    const size_t per_chunk = static_cast<size_t>(p.B) * p.D * nch * sizeof(float);
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    char* ws = static_cast<char*>(workspace);
    BwdWork w{};
    w.want_fwd = chunk_states == nullptr;
    w.fill = fill;
    w.spin_limit = ring_spin_limit();
    // the trapezoidal rule has no fused pass: its plan is the one that fits in no bytes
    const BwdPlan plan =
        bwd_plan(p.B, p.D, p.N, p.L, w.want_fwd, p.lam != nullptr ? 0 : workspace_bytes);
    if (plan.bytes > workspace_bytes) return hipErrorInvalidValue;
    const Timing tm{ev_begin, ev_end};
    if (plan.fused) {
        w.H = const_cast<float*>(chunk_states);
        w.G = reinterpret_cast<float*>(ws);
        ws += up(static_cast<size_t>(p.B) * p.D * p.N * sizeof(float));
        w.part = reinterpret_cast<float*>(ws);
        ws += up(static_cast<size_t>(p.B) * plan.cgroups * nch * 2 * p.N * kChunk *
                 sizeof(float));
        w.dApart = reinterpret_cast<float*>(ws);
        ws += up(states);
        w.dDpart = reinterpret_cast<float*>(ws);
        ws += up(per_chunk);
        w.dbpart = reinterpret_cast<float*>(ws);
    } else {
        if (w.want_fwd) {
            w.H = reinterpret_cast<float*>(ws);
            ws += up(states);
        } else {
            w.H = const_cast<float*>(chunk_states);
        }
        w.G = reinterpret_cast<float*>(ws);
        ws += up(states);
        w.sdt = reinterpret_cast<float*>(ws);
        ws += up(per_chunk);
        w.dfirst = reinterpret_cast<float*>(ws);
        w.c0 = (!w.want_fwd && g.dh0 == nullptr) ? 1 : 0;
    }
    if (bf16) return bwd_dispatch<bf16_t>(p, g, w, plan, stream, tm);
    return bwd_dispatch<float>(p, g, w, plan, stream, tm);
}

MSEL_BOUNDS_TAKER(take_bounds_bwd)

}  // namespace msel
