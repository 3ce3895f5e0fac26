// scan_cplx_bwd.hip -- backward of the complex-valued (rotational) scan, with recomputation.
//
// The forward (scan_cplx.hip; page 5, the Mamba-3 post, second bullet) runs, per state pair j of
// channel d, the complex recurrence h_t = a_t h_{t-1} + Delta_t u_t B_t with a_t =
// exp(Delta_t (A_re + i A_im)), B_t = B_{2j,t} + i B_{2j+1,t}, and reads out
// y_t = Re(conj(C_t) h_t) + D u_t with C_t = C_{2j,t} + i C_{2j+1,t}.  With G_t the adjoint
// dL/dRe h_t + i dL/dIm h_t (page 1; page 4 Appendix D, Memory: states are recomputed, not
// stored):
//   G_t = C_t dy_t + conj(a_{t+1}) G_{t+1}               (zero beyond the last step)
//   dB_t += Delta_t u_t G_t      dC_t += dy_t h_t      (real and imaginary parts, summed
//                                                         over channels)
//   X_t = conj(G_t) a_t h_{t-1}:  dDelta_t += Re(A X_t),  dA_re += Delta_t Re X_t,
//                                 dA_im -= Delta_t Im X_t
//   du_t = Delta_t Re(conj(G_t) B_t) + D dy_t,  dDelta_t += u_t Re(conj(G_t) B_t)
//   dh0 = conj(a_0) G_0
//
// Three launches, as for the real scan, from the forward's chunk states:
//  1. summary: one wavefront per (batch, chunk, channel): per pair the adjoint at the chunk's
//     first step from the chunk alone, sum_t exp(conj(A) E_t) C_t dy_t (E_t: sum of Delta
//     over the chunk's steps 1..t), plus sum(Delta) and Delta at the first step;
//  2. link: one thread per (batch, channel, pair) walks the chunks backwards,
//     G_{c-1} = conj(exp(A sum Delta_c)) G_c + conj(exp(A Delta_first_c)) Sr_c;
//  3. gradient kernel: one workgroup per (batch, chunk, range of channels), one wavefront per
//     channel, the pairs walked in ring order over shared LDS accumulators for dB and dC (the
//     real scan's gradient kernel, with complex pairs for states).  Per pair it rebuilds the
//     states (lane chains + complex affine DPP scan from H_c) and the adjoints (reverse lane
//     chains + complex suffix scan from G_c) and forms every term; the per-token sums over
//     pairs (for du, dDelta and the gated y) stay in the wavefront's registers.
#include "msel_device.hpp"
#include "msel_kernels.hpp"

namespace msel {

namespace {

constexpr int kK = kChunk / 64;  // steps per lane
constexpr int kMaxPairs = 8;

struct CWork {
    const float* H;  // [B*D*nch*N]: chunk-start states (the forward's chunk_states)
    float* G;        // [B*D*nch*N]: per chunk the local adjoint, then the adjoint carry
    float* sdt;      // [B*D*nch]: sum of Delta over the chunk
    float* dfirst;   // [B*D*nch]: Delta at the chunk's first step
    int c0;          // first chunk summarised: chunk 0's summary feeds only dh0, so it is
                     // skipped (c0 = 1) when dh0 is not asked for
    FillList fill;   // the gradient kernel's reduction targets, zeroed by the link launch
    unsigned spin_limit;  // polls after which a ring wait gives up (ring_spin_limit())
};

// Ring waits of this file's gradient kernel that gave up (see ring_spin_limit).
__device__ unsigned long long g_ring_timeouts_cplx;

// ---------------------------------------------------------------------------------------
// 1. summary

template <typename T, bool VEC, bool HAS_Z, bool SOFTPLUS>
__global__ __launch_bounds__(256) void cplx_summary_kernel(ScanParams p, GradParams g, CWork w) {
    constexpr int K = kK;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int nch = p.nchunks;
    const int nsum = nch - w.c0;  // chunks summarised
    const long long unit = static_cast<long long>(blockIdx.x) * 4 + wave;  // (b, c - c0, d)
    if (unit >= static_cast<long long>(p.B) * nsum * p.D) return;
    const int d = static_cast<int>(unit % p.D);
    const int c = w.c0 + static_cast<int>((unit / p.D) % nsum);
    const int b = static_cast<int>(unit / (static_cast<long long>(p.D) * nsum));
    const int L = p.L, N = p.N;
    [[maybe_unused]] const size_t BD = static_cast<size_t>(p.B) * p.D;
    const size_t ch = MSEL_IDX(static_cast<size_t>(b) * p.D + d, BD);
    const size_t row = ch * L;
    const int t0 = c * kChunk + lane * K;
    const float bias = p.bias ? p.bias[MSEL_IDX(d, p.D)] : 0.0f;

    float dt[K], dy[K];
    {
        float dd[K], go[K];
        load_k_cached<T, K, VEC>(static_cast<const T*>(p.delta) + row, t0, L, dd);
        load_k_cached<T, K, VEC>(static_cast<const T*>(g.dout) + row, t0, L, go);
        float zz[HAS_Z ? K : 1];
        if constexpr (HAS_Z) load_k_cached<T, K, VEC>(static_cast<const T*>(p.z) + row, t0, L, zz);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float x = dd[k] + bias;
            const float v = SOFTPLUS ? softplus_f(x) : x;
            dt[k] = (t0 + k < L) ? v : 0.0f;
            dy[k] = HAS_Z ? go[k] * zz[k] * sigmoid_f(zz[k]) : go[k];
        }
    }
    // E_t: sum of Delta over the chunk's steps 1..t, summed from those steps alone (the first
    // step left out of the running sum, not subtracted: next to a reset step's huge Delta a
    // difference of two sums would keep only a few bits of E_t)
    float E[K];
    float run = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        run += (k == 0 && lane == 0) ? 0.0f : dt[k];
        E[k] = run;
    }
    const float incl = wave_incl_sum(run);
    const float before = shift_up(incl, 0.0f);      // Delta of the lanes before this one
    const float first = readlane(dt[0], 0);          // Delta at the chunk's first step
    const float total = readlane(incl, 63) + first;
#pragma unroll
    for (int k = 0; k < K; ++k) E[k] += before;

    const T* __restrict__ Cg =
        static_cast<const T*>(p.Cm) + static_cast<size_t>(MSEL_IDX(b, p.B)) * N * L;
    const float* Ad = p.A + static_cast<size_t>(MSEL_IDX(d, p.D)) * N;
    float outv = 0.0f;  // lane n: component n of the summary
    for (int n = 0; n < N; n += 4) {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // (re, im) of pairs n/2 and n/2 + 1
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int m = n + 2 * q;
            if (m >= N) break;
            const float Ar = Ad[MSEL_IDX(m, N)] * kLog2e, Ai = Ad[MSEL_IDX(m + 1, N)] * kInv2Pi;
            float cr[K], ci[K];
            load_k_cached<T, K, VEC>(Cg + static_cast<size_t>(MSEL_IDX(m, N)) * L, t0, L, cr);
            load_k_cached<T, K, VEC>(Cg + static_cast<size_t>(MSEL_IDX(m + 1, N)) * L, t0, L, ci);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                // exp(conj(A) E) C dy
                const float e = exp2_hw(Ar * E[k]) * dy[k];
                const float co = cos_rev(Ai * E[k]), si = sin_rev(Ai * E[k]);
                acc[2 * q] = fmaf(e, fmaf(co, cr[k], si * ci[k]), acc[2 * q]);
                acc[2 * q + 1] = fmaf(e, fmaf(co, ci[k], -si * cr[k]), acc[2 * q + 1]);
            }
        }
        wave_sum4(acc[0], acc[1], acc[2], acc[3]);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (n + q < N) outv = writelane(acc[q], n + q, outv);
    }
    const size_t base = MSEL_IDX(ch * nch + c, BD * nch);
    if (lane < N) w.G[MSEL_IDX(base * N + lane, BD * nch * N)] = outv;
    if (lane == 0) {
        w.sdt[base] = total;
        w.dfirst[base] = first;
    }
}

// ---------------------------------------------------------------------------------------
// 2. link

// One thread per (batch, channel, pair); the launch also zeroes the gradient kernel's reduction
// targets (its grid may be wider than the links for that).
__global__ __launch_bounds__(256) void cplx_link_kernel(ScanParams p, GradParams g, CWork w) {
    const int J = p.N / 2;
    const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
    zero_fill(w.fill, static_cast<size_t>(i), static_cast<size_t>(gridDim.x) * blockDim.x);
    if (i >= static_cast<long long>(p.B) * p.D * J) return;
    const long long ch = i / J;
    const int j = static_cast<int>(i - ch * J);
    const int d = static_cast<int>(ch % p.D);
    const int nch = p.nchunks;
    [[maybe_unused]] const size_t DN = static_cast<size_t>(p.D) * p.N;
    [[maybe_unused]] const size_t BDC = static_cast<size_t>(p.B) * p.D * nch;
    const float Ar = p.A[MSEL_IDX(static_cast<size_t>(d) * p.N + 2 * j, DN)] * kLog2e;
    const float Ai = p.A[MSEL_IDX(static_cast<size_t>(d) * p.N + 2 * j + 1, DN)] * kInv2Pi;
    float Gr = 0.0f, Gi = 0.0f;
    for (int c = nch - 1; c >= w.c0; --c) {
        const size_t base = MSEL_IDX(static_cast<size_t>(ch) * nch + c, BDC);
        float* slot = w.G + base * p.N + MSEL_IDX(2 * j, p.N - 1);  // slot[0], slot[1]
        const float Sr = slot[0], Si = slot[1];
        slot[0] = Gr;
        slot[1] = Gi;
        const float s = w.sdt[base], f = w.dfirst[base];
        // conj(exp(A s)) G + conj(exp(A f)) S
        const float es = exp2_hw(Ar * s), ef = exp2_hw(Ar * f);
        const float cs = es * cos_rev(Ai * s), ss = -es * sin_rev(Ai * s);
        const float cf = ef * cos_rev(Ai * f), sf = -ef * sin_rev(Ai * f);
        float ar, ai, br, bi;
        cmul(cs, ss, Gr, Gi, ar, ai);
        cmul(cf, sf, Sr, Si, br, bi);
        Gr = ar + br;
        Gi = ai + bi;
    }
    if (w.c0 > 0) {  // the carry after chunk 0 (no summary of its own)
        float* slot = w.G + static_cast<size_t>(ch) * nch * p.N + MSEL_IDX(2 * j, p.N - 1);
        slot[0] = Gr;
        slot[1] = Gi;
    }
    if (g.dh0 != nullptr) {
        g.dh0[static_cast<size_t>(ch) * p.N + MSEL_IDX(2 * j, p.N - 1)] = Gr;
        g.dh0[static_cast<size_t>(ch) * p.N + MSEL_IDX(2 * j, p.N - 1) + 1] = Gi;
    }
}

// ---------------------------------------------------------------------------------------
// 3. gradient kernel
//
// One workgroup per (batch row, chunk, range of channels), one wavefront per channel at a
// time, the state pairs walked in ring order: at global step s (channel round * J + step) the
// wave `rot` of a group of J waves works on pair (rot + s) mod J.  The chunk's B and C sit in
// LDS as fp32 for all waves; each group sums its channels' dB and dC in LDS accumulator rows
// shared by its waves, and the per-token sums over pairs (for du, dDelta and the gated y)
// stay in the wave's registers, so no workgroup barrier is needed between channels.  The
// previous update of pair (rot + s) mod J was made one step earlier by wave rot + 1 (by wave
// 0 for the group's last wave): a wave publishes every step it finishes in the pair's flag,
// and the next writer of that pair waits for it.  Every wave runs every step (inactive ones
// only publish), the chain ends at step 0, and all waves of a workgroup are resident, so
// the waits end.

constexpr int kRingWaves = 8;     // at most; a workgroup has J * (kRingWaves / J) waves
constexpr int kRingKP = 65;       // padded stride of the accumulator rows (conflict-free)
constexpr int kRingQuads = 16;    // dA partials per (wave, component): sums of 4 lanes
constexpr int kMaxRingFlags = kRingWaves;

__host__ __device__ constexpr int ring_waves(int J) { return J * (kRingWaves / J); }

// dB and dC accumulators [2][groups][N][K][KP], the chunk's B and C [2][N][kChunk] (fp32),
// the per-wave dA partials [W][N][kRingQuads]
__host__ __device__ constexpr size_t ring_lds_bytes(int N) {
    return (2 * static_cast<size_t>(kRingWaves / (N / 2)) * N * kK * kRingKP +
            2 * static_cast<size_t>(N) * kChunk +
            static_cast<size_t>(ring_waves(N / 2)) * N * kRingQuads) *
           sizeof(float);
}
__host__ __device__ constexpr size_t ring_lds_bytes_max() {
    size_t m = 0;
    for (int n = 2; n <= 2 * kMaxPairs; n += 2) m = ring_lds_bytes(n) > m ? ring_lds_bytes(n) : m;
    return m;
}
static_assert(ring_lds_bytes_max() + kMaxRingFlags * sizeof(int) +
                      static_cast<size_t>(kRingWaves) * kMaxN * 16 <= 160 * 1024,
              "complex gradient kernel LDS exceeds a compute unit's 160 KB");

template <typename T, bool VEC, bool HAS_Z, bool SOFTPLUS>
__global__ __launch_bounds__(64 * kRingWaves) void cplx_main_kernel(ScanParams p, GradParams g,
                                                                    CWork w, int per_wave) {
    constexpr int K = kK;
    constexpr int KP = kRingKP;
    // bf16 rows are small enough that the next channel's u and delta are fetched during the
    // current channel's last step, next to this channel's z and dout (for dz)
    constexpr bool kEarlyUD = sizeof(T) == 2;
    extern __shared__ float acc[];
    __shared__ int ring_flags[kMaxRingFlags];
    // Per wavefront and state component, the channel's A, A scaled for exp2 (Re: log2(e)) or
    // in revolutions (Im: 1 / (2 pi)), H_c and G_c: written once per channel by lane n, read
    // per step with broadcast LDS reads instead of v_readlane's.
    __shared__ f32x4 ccells[kRingWaves][kMaxN];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int W = static_cast<int>(blockDim.x >> 6);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // one-dimensional grid over (batch row, chunk, channel group), channel groups fastest
    const int cgroups = static_cast<int>(gridDim.x) / (p.B * p.nchunks);
    const int bc_ = static_cast<int>(blockIdx.x) / cgroups;
    const int cgrp = static_cast<int>(blockIdx.x) - bc_ * cgroups;
    const int b = bc_ / p.nchunks;
    const int c = bc_ - b * p.nchunks;
    const int N = p.N;
    const int J = N / 2;
    const int L = p.L;
    const int nch = p.nchunks;
    const int groups = W / J;
    const int tile = N * K * KP;  // floats per (tensor, group)
    float* accB = acc;
    float* accC = acc + groups * tile;
    float* BCs = acc + 2 * groups * tile;                            // B rows, then C rows
    float* dAs = BCs + 2 * N * kChunk + wave * N * kRingQuads;     // this wave's dA partials
    for (int i = tid; i < 2 * groups * tile; i += 64 * W) acc[i] = 0.0f;
    for (int i = tid; i < groups * J; i += 64 * W) ring_flags[MSEL_IDX(i, kMaxRingFlags)] = 0;
    [[maybe_unused]] const size_t BD = static_cast<size_t>(p.B) * p.D;
    [[maybe_unused]] const size_t DN = static_cast<size_t>(p.D) * N;
    {
        // B and C of this (batch row, chunk), read once per workgroup, zero past the end;
        // lane l's 8 steps of a row are two 16-byte vectors, consecutive lanes adjacent
        const T* __restrict__ Bg =
            static_cast<const T*>(p.Bm) + static_cast<size_t>(MSEL_IDX(b, p.B)) * N * L;
        const T* __restrict__ Cg =
            static_cast<const T*>(p.Cm) + static_cast<size_t>(MSEL_IDX(b, p.B)) * N * L;
        for (int i = tid; i < N * kChunk; i += 64 * W) {
            const int nn = i / kChunk;
            const int tl = i - nn * kChunk;
            const int t = c * kChunk + tl;
            float vb = 0.0f, vc = 0.0f;
            if (t < L) {
                vb = Elem<T>::load1(Bg + static_cast<size_t>(nn) * L + t);
                vc = Elem<T>::load1(Cg + static_cast<size_t>(nn) * L + t);
            }
            const int o = MSEL_IDX(((nn * 2 + (tl % K) / 4) * 64 + tl / K) * 4 + tl % 4,
                                   N * kChunk);
            BCs[o] = vb;
            BCs[N * kChunk + o] = vc;
        }
    }
    __syncthreads();

    const int grp = wave / J;
    const int rot = wave - grp * J;
    int* gflags = ring_flags + MSEL_IDX(grp * J, kMaxRingFlags);
    int gstep = 0;
    float* myB = accB + grp * tile;
    float* myC = accC + grp * tile;

    const int t0 = c * kChunk + lane * K;
    const f32x4* __restrict__ B4 = reinterpret_cast<const f32x4*>(BCs);
    const f32x4* __restrict__ C4 = reinterpret_cast<const f32x4*>(BCs + N * kChunk);
    const T* __restrict__ gu = static_cast<const T*>(p.u);
    const T* __restrict__ gd = static_cast<const T*>(p.delta);
    const T* __restrict__ gg_ = static_cast<const T*>(g.dout);
    const T* __restrict__ gz = static_cast<const T*>(p.z);
    auto chan_row = [&](int d) { return MSEL_IDX(static_cast<size_t>(b) * p.D + d, BD) * L; };

    // raw input rows of the channel about to start, fetched ahead of time
    Raw<T, K> ru, rd, rg, rz;
    const int d_first = cgrp * per_wave * W + wave;
    if (d_first < p.D) {
        const size_t row = chan_row(d_first);
        load_raw<T, K, VEC>(gu + row, t0, L, ru);
        load_raw<T, K, VEC>(gd + row, t0, L, rd);
        load_raw<T, K, VEC>(gg_ + row, t0, L, rg);
        if constexpr (HAS_Z) load_raw<T, K, VEC>(gz + row, t0, L, rz);
    }

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
        // per-channel rows of A, H_c and G_c, one component per lane ((Re, Im) interleaved)
        const size_t hg = (ch * nch + c) * N;
        const float Av = (lane < N) ? p.A[MSEL_IDX(static_cast<size_t>(dd_) * N + lane, DN)] : 0.0f;
        const float Hv = (lane < N) ? w.H[MSEL_IDX(hg + lane, BD * nch * N)] : 0.0f;
        const float Gv = (lane < N) ? w.G[MSEL_IDX(hg + lane, BD * nch * N)] : 0.0f;
        if (lane < N) ccells[wave][lane] = f32x4{Av, Av * ((lane & 1) ? kInv2Pi : kLog2e), Hv, Gv};

        int jn = rot;  // pair of step 0

        float dt[K], dtu[K], dy[K], sB[K], sgA[K];
        // HAS_Z: y for dz, and dz's factor dout * silu'(z) = dout s (1 + z (1 - s)), formed
        // here beside dy with the same sigmoid s
        float y[HAS_Z ? K : 1], fz[HAS_Z ? K : 1];
        float sum_dt = 0.0f, dD_part = 0.0f;
        {
            float uu[K], dd[K], go[K];
            unpack(ru, uu);
            unpack(rd, dd);
            unpack(rg, go);
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
                dtu[k] = dt[k] * uu[k];
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
        }

        auto step = [&](const bool last) __attribute__((always_inline)) {
            const int jc = jn;
            const int n0 = 2 * jc;
            // the pair's A, scaled A, H_c and G_c: (Re) component n0 and (Im) n0 + 1
            const f32x4 cre = ccells[wave][MSEL_IDX(n0, kMaxN - 1)];
            const f32x4 cim = ccells[wave][MSEL_IDX(n0, kMaxN - 1) + 1];
            float Br[K], Bi[K], Cr[K], Ci[K];
            {
                [[maybe_unused]] const int NW = N * kChunk / 4;  // 16-byte words per tensor
                const f32x4 b0 = B4[MSEL_IDX((n0 * 2) * 64 + lane, NW)],
                            b1 = B4[MSEL_IDX((n0 * 2 + 1) * 64 + lane, NW)];
                const f32x4 b2 = B4[MSEL_IDX((n0 * 2 + 2) * 64 + lane, NW)],
                            b3 = B4[MSEL_IDX((n0 * 2 + 3) * 64 + lane, NW)];
                const f32x4 c0 = C4[MSEL_IDX((n0 * 2) * 64 + lane, NW)],
                            c1 = C4[MSEL_IDX((n0 * 2 + 1) * 64 + lane, NW)];
                const f32x4 c2 = C4[MSEL_IDX((n0 * 2 + 2) * 64 + lane, NW)],
                            c3 = C4[MSEL_IDX((n0 * 2 + 3) * 64 + lane, NW)];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    Br[q] = b0[q];
                    Br[4 + q] = b1[q];
                    Bi[q] = b2[q];
                    Bi[4 + q] = b3[q];
                    Cr[q] = c0[q];
                    Cr[4 + q] = c1[q];
                    Ci[q] = c2[q];
                    Ci[4 + q] = c3[q];
                }
            }
            if (!last) {
                jn = (jn + 1 == J) ? 0 : jn + 1;
            } else {
                // no branches around these loads: for a channel that is not there they start
                // past the row's end (zeros, no memory access), so that the waits for them
                // count exactly the loads issued after them
                if constexpr (kEarlyUD) {
                    load_raw<T, K, VEC>(gu + row_next, next_active ? t0 : L, L, ru);
                    load_raw<T, K, VEC>(gd + row_next, next_active ? t0 : L, L, rd);
                }
            }
            // wait until the previous update of pair jc (one step earlier) is complete
            if (gstep > 0) {
                unsigned polls = 0;
                while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(
                           gflags + MSEL_IDX(jc, kMaxRingFlags - grp * J), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP)) < gstep) {
                    if (++polls >= w.spin_limit) {  // give up: counted, never a hang
                        if (lane == 0)
                            __hip_atomic_fetch_add(&g_ring_timeouts_cplx, 1ull, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            asm volatile("" ::: "memory");
            if (active) {
                // rows k of the pair's two components are sBr[k * KP], sBi[k * KP] (the
                // base's extent leaves room for both and the 64 lanes)
                float* sBr = myB + MSEL_IDX(n0 * K * KP, tile - (2 * K - 1) * KP - 63) + lane;
                float* sBi = sBr + K * KP;
                float* sCr = myC + MSEL_IDX(n0 * K * KP, tile - (2 * K - 1) * KP - 63) + lane;
                float* sCi = sCr + K * KP;
                float ocr[K], oci[K];
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    ocr[k] = sCr[k * KP];
                    oci[k] = sCi[k * KP];
                }
                const float ArRaw = cre[0], AiRaw = cim[0];
                const float Ar = cre[1], Ai = cim[1];
                const float Hr = cre[2], Hi = cim[2];
                const float Gr = cre[3], Gi = cim[3];

                // pass 1: transitions, the lane chain of states from zero, and the lane chain
                // of adjoints from a zero input on the right
                float ar[K], ai[K], bbr[K], bbi[K];
                float hr = 0.0f, hi = 0.0f;
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const float e = exp2_hw(dt[k] * Ar);
                    const float rv = dt[k] * Ai;
                    ar[k] = e * cos_rev(rv);
                    ai[k] = e * sin_rev(rv);
                    bbr[k] = dtu[k] * Br[k];
                    bbi[k] = dtu[k] * Bi[k];
                    const float nr = fmaf(ar[k], hr, fmaf(-ai[k], hi, bbr[k]));
                    hi = fmaf(ai[k], hr, fmaf(ar[k], hi, bbi[k]));
                    hr = nr;
                }
                float gr = dy[K - 1] * Cr[K - 1], gi = dy[K - 1] * Ci[K - 1];
#pragma unroll
                for (int k = K - 2; k >= 0; --k) {
                    const float tr = fmaf(ar[k + 1], gr, ai[k + 1] * gi);
                    const float ti = fmaf(ar[k + 1], gi, -ai[k + 1] * gr);
                    gr = fmaf(dy[k], Cr[k], tr);
                    gi = fmaf(dy[k], Ci[k], ti);
                }
                // lane maps: states, x -> P x + S with P = a_{K-1} ... a_0 = exp(A sum_dt);
                // adjoints, from the one arriving on the right (carried into the lane's last
                // step) to the one leaving on the left, x -> conj(a_0) (g_0 + conj(a_{K-1}
                // ... a_1) x) = conj(P) x + conj(a_0) g_0
                const float eP = exp2_hw(sum_dt * Ar), rP = sum_dt * Ai;
                float Pr = eP * cos_rev(rP), Pi = eP * sin_rev(rP), Sr = hr, Si = hi;
                float Rr = Pr, Ri = -Pi, Tr, Ti;
                cmul(ar[0], -ai[0], gr, gi, Tr, Ti);
                cscan2_fused(Pr, Pi, Sr, Si, Rr, Ri, Tr, Ti);
                float hin_r, hin_i;  // the state entering the lane
                {
                    float tr, ti;
                    cmul(Pr, Pi, Hr, Hi, tr, ti);
                    hin_r = shift_up(tr + Sr, Hr);
                    hin_i = shift_up(ti + Si, Hi);
                }
                // the adjoint arriving on the right of each 16-lane row, from G_c through the
                // rows after it
                float Er[4], Ei[4];
                Er[3] = Gr;
                Ei[3] = Gi;
#pragma unroll
                for (int q = 3; q > 0; --q) {
                    const float pr = readlane(Rr, 16 * q), pi = readlane(Ri, 16 * q);
                    const float sr = readlane(Tr, 16 * q), si = readlane(Ti, 16 * q);
                    float tr, ti;
                    cmul(pr, pi, Er[q], Ei[q], tr, ti);
                    Er[q - 1] = tr + sr;
                    Ei[q - 1] = ti + si;
                }
                const int myrow = lane >> 4;
                const float er = myrow == 0 ? Er[0] : myrow == 1 ? Er[1] : myrow == 2 ? Er[2] : Er[3];
                const float ei = myrow == 0 ? Ei[0] : myrow == 1 ? Ei[1] : myrow == 2 ? Ei[2] : Ei[3];
                float gin_r, gin_i;  // the adjoint arriving on this lane's right
                {
                    float tr, ti;
                    cmul(Rr, Ri, er, ei, tr, ti);
                    gin_r = shift_down(tr + Tr, Gr);
                    gin_i = shift_down(ti + Ti, Gi);
                }

                // pass 2: states, y and dC
                float hsr[K], hsi[K];
                hr = hin_r;
                hi = hin_i;
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const float nr = fmaf(ar[k], hr, fmaf(-ai[k], hi, bbr[k]));
                    hi = fmaf(ai[k], hr, fmaf(ar[k], hi, bbi[k]));
                    hr = nr;
                    hsr[k] = hr;
                    hsi[k] = hi;
                    if constexpr (HAS_Z) y[k] = fmaf(Cr[k], hr, fmaf(Ci[k], hi, y[k]));
                    ocr[k] = fmaf(dy[k], hr, ocr[k]);
                    oci[k] = fmaf(dy[k], hi, oci[k]);
                }
                float obr[K], obi[K];
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    sCr[k * KP] = ocr[k];
                    sCi[k * KP] = oci[k];
                    obr[k] = sBr[k * KP];
                    obi[k] = sBi[k * KP];
                }
                // reverse pass: the adjoint at every step and the gradient terms
                float dAr = 0.0f, dAi = 0.0f;
                gr = gin_r;
                gi = gin_i;
#pragma unroll
                for (int k = K - 1; k >= 0; --k) {
                    if (k < K - 1) {
                        const float tr = fmaf(ar[k + 1], gr, ai[k + 1] * gi);
                        const float ti = fmaf(ar[k + 1], gi, -ai[k + 1] * gr);
                        gr = tr;
                        gi = ti;
                    }
                    gr = fmaf(dy[k], Cr[k], gr);
                    gi = fmaf(dy[k], Ci[k], gi);
                    obr[k] = fmaf(gr, dtu[k], obr[k]);
                    obi[k] = fmaf(gi, dtu[k], obi[k]);
                    sB[k] = fmaf(gr, Br[k], fmaf(gi, Bi[k], sB[k]));
                    const float pr = (k == 0) ? hin_r : hsr[k - 1];
                    const float pi = (k == 0) ? hin_i : hsi[k - 1];
                    float ahr, ahi;
                    cmul(ar[k], ai[k], pr, pi, ahr, ahi);
                    // X = conj(g) a h_prev
                    const float Xr = fmaf(gr, ahr, gi * ahi), Xi = fmaf(gr, ahi, -gi * ahr);
                    sgA[k] = fmaf(ArRaw, Xr, fmaf(-AiRaw, Xi, sgA[k]));
                    dAr = fmaf(dt[k], Xr, dAr);
                    dAi = fmaf(-dt[k], Xi, dAi);
                }
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    sBr[k * KP] = obr[k];
                    sBi[k * KP] = obi[k];
                }
                const float qr = quad_sum(dAr), qi = quad_sum(dAi);
                if ((lane & 3) == 0) {
                    dAs[MSEL_IDX(n0 * kRingQuads + (lane >> 2), N * kRingQuads)] = qr;
                    dAs[MSEL_IDX((n0 + 1) * kRingQuads + (lane >> 2), N * kRingQuads)] = qi;
                }
            }
            // publish: this step's LDS writes are complete
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __hip_atomic_store(gflags + MSEL_IDX(jc, kMaxRingFlags - grp * J), gstep + 1,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            ++gstep;
        };

        for (int q = 0; q + 1 < J; ++q) step(false);
        step(true);

        // this channel's u and delta again (its rows, still in L2), issued before the next
        // channel's loads so that waiting for them does not wait for those (and, as in the last
        // step, without branches)
        Raw<T, K> ruu;
        [[maybe_unused]] Raw<T, K> rxs;
        load_raw<T, K, VEC>(gu + row, active ? t0 : L, L, ruu);
        if constexpr (SOFTPLUS) load_raw<T, K, VEC>(gd + row, active ? t0 : L, L, rxs);
        asm volatile("" ::: "memory");  // keep them ahead of the loads below
        // the rest of the next channel's inputs, in flight while this one is finished
        {
            const int tn = next_active ? t0 : L;
            if constexpr (!kEarlyUD) {
                load_raw<T, K, VEC>(gu + row_next, tn, L, ru);
                load_raw<T, K, VEC>(gd + row_next, tn, L, rd);
            }
            load_raw<T, K, VEC>(gg_ + row_next, tn, L, rg);
            if constexpr (HAS_Z) load_raw<T, K, VEC>(gz + row_next, tn, L, rz);
        }
        if (!active) continue;

        // du, ddelta and dz; with the softplus, ddelta = dDelta * sigmoid(delta + bias), formed
        // from delta + bias and Delta (softplus_grad_f).
        float uu[K];
        unpack(ruu, uu);
        float xs[SOFTPLUS ? K : 1];  // delta + bias
        if constexpr (SOFTPLUS) {
            unpack(rxs, xs);
#pragma unroll
            for (int k = 0; k < K; ++k) xs[k] += bias;
        }
        float o1[K], o2[K];
        float db_part = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float dsp = SOFTPLUS ? softplus_grad_f(xs[k], dt[k]) : 1.0f;
            o1[k] = fmaf(sB[k], dt[k], dy[k] * Dd);        // du
            o2[k] = fmaf(sB[k], uu[k], sgA[k]) * dsp;     // ddelta
        }
        if ((c + 1) * kChunk > L) {  // dbias: past-the-end steps masked in a ragged chunk only
#pragma unroll
            for (int k = 0; k < K; ++k) db_part += (t0 + k < L) ? o2[k] : 0.0f;
        } else {
#pragma unroll
            for (int k = 0; k < K; ++k) db_part += o2[k];
        }
        store_k<T, K, VEC>(static_cast<T*>(g.du) + row, t0, L, o1);
        store_k<T, K, VEC>(static_cast<T*>(g.ddelta) + row, t0, L, o2);
        if constexpr (HAS_Z) {  // dz = dout * y * silu'(z), y complete over every pair
            float o3[K];
#pragma unroll
            for (int k = 0; k < K; ++k) o3[k] = fz[k] * y[k];
            store_k<T, K, VEC>(static_cast<T*>(g.dz) + row, t0, L, o3);
        }
        // dA[d, n]: lane n sums the quad partials of component n (the wave's own rows: same-
        // wave LDS order, no barrier needed)
        float sa = 0.0f;
        if (lane < N) {
            const f32x4* src = reinterpret_cast<const f32x4*>(
                dAs + MSEL_IDX(lane * kRingQuads, N * kRingQuads));
#pragma unroll
            for (int q = 0; q < kRingQuads / 4; ++q) {
                const f32x4 v = src[q];
                sa += (v[0] + v[1]) + (v[2] + v[3]);
            }
        }
        const float sD = wave_sum_fused(dD_part);
        const float sb = wave_sum_fused(db_part);
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

    // this workgroup's share of dB and dC
    __syncthreads();
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
}

template <typename T, bool VEC, bool HAS_Z, bool SP>
hipError_t cplx_bwd_go(const ScanParams& p, const GradParams& g, const CWork& w,
                       hipStream_t s) {
    const long long units = static_cast<long long>(p.B) * (p.nchunks - w.c0) * p.D;
    hipError_t e = hipSuccess;
    if (units > 0) {  // none with a single chunk and no dh0
        hipLaunchKernelGGL((cplx_summary_kernel<T, VEC, HAS_Z, SP>),
                           dim3(static_cast<unsigned>((units + 3) / 4)), dim3(256), 0, s, p, g,
                           w);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const long long links = static_cast<long long>(p.B) * p.D * (p.N / 2);
    hipLaunchKernelGGL(cplx_link_kernel,
                       dim3(std::max(static_cast<unsigned>((links + 255) / 256),
                                     fill_blocks(w.fill))),
                       dim3(256), 0, s, p, g, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // channels per wavefront: about one workgroup per compute unit over (batch, chunk,
    // channel ranges), so that each flushes its dB / dC sums once for many channels
    const int cus = device_compute_units();
    const int W = ring_waves(p.N / 2);
    const long long slots = static_cast<long long>(p.B) * p.nchunks;
    long long per = (static_cast<long long>(p.D) * slots + static_cast<long long>(cus) * W - 1) /
                    (static_cast<long long>(cus) * W);
    const long long max_per = (p.D + W - 1) / W;
    if (per < 1) per = 1;
    if (per > max_per) per = max_per;
    const int cgroups = static_cast<int>((p.D + per * W - 1) / (per * W));
    // the LDS exceeds the 64 KB default; allow the largest need over the pair counts
    const hipError_t attr = allow_dynamic_lds<&cplx_main_kernel<T, VEC, HAS_Z, SP>>(
        static_cast<int>(ring_lds_bytes_max()));
    if (attr != hipSuccess) return attr;
    const long long mblocks = static_cast<long long>(cgroups) * p.nchunks * p.B;
    if (mblocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((cplx_main_kernel<T, VEC, HAS_Z, SP>), dim3(static_cast<unsigned>(mblocks)),
                       dim3(64 * W), ring_lds_bytes(p.N), s, p, g, w, static_cast<int>(per));
    return hipGetLastError();
}

template <typename T>
hipError_t cplx_bwd_dispatch(const ScanParams& p, const GradParams& g, const CWork& w,
                             hipStream_t s) {
    const bool vec = (static_cast<size_t>(p.L) * sizeof(T)) % 16 == 0;
    const bool hz = p.z != nullptr, sp = p.softplus != 0;
#define MSEL_CB(V, Z, S) \
    if (vec == V && hz == Z && sp == S) return cplx_bwd_go<T, V, Z, S>(p, g, w, s);
    MSEL_CB(true, true, true)
    MSEL_CB(true, true, false)
    MSEL_CB(true, false, true)
    MSEL_CB(true, false, false)
    MSEL_CB(false, true, true)
    MSEL_CB(false, true, false)
    MSEL_CB(false, false, true)
    MSEL_CB(false, false, false)
#undef MSEL_CB
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t take_ring_timeouts_cplx(unsigned long long* count) {
    unsigned long long v = 0;
    const unsigned long long zero = 0;
    hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_ring_timeouts_cplx), sizeof(v), 0,
                                       hipMemcpyDeviceToHost);
    if (e == hipSuccess)
        e = hipMemcpyToSymbol(HIP_SYMBOL(g_ring_timeouts_cplx), &zero, sizeof(zero), 0,
                              hipMemcpyHostToDevice);
    *count = v;
    return e;
}

hipError_t launch_scan_cplx_bwd(const ScanParams& p, const GradParams& g,
                                const float* chunk_states, void* workspace, bool bf16,
                                const FillList& fill, hipStream_t stream) {
    if (p.N % 2 != 0 || p.N > 2 * kMaxPairs || chunk_states == nullptr)
        return hipErrorInvalidValue;
    const size_t nch = static_cast<size_t>(p.nchunks);
    const size_t states = static_cast<size_t>(p.B) * p.D * nch * p.N * sizeof(float);
    const size_t per_chunk = static_cast<size_t>(p.B) * p.D * nch * sizeof(float);
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    char* ws = static_cast<char*>(workspace);
    CWork w;
    w.H = chunk_states;
    w.G = reinterpret_cast<float*>(ws);
    ws += up(states);
    w.sdt = reinterpret_cast<float*>(ws);
    ws += up(per_chunk);
    w.dfirst = reinterpret_cast<float*>(ws);
    w.c0 = g.dh0 == nullptr ? 1 : 0;
    w.fill = fill;
    w.spin_limit = ring_spin_limit();
    return bf16 ? cplx_bwd_dispatch<bf16_t>(p, g, w, stream)
                : cplx_bwd_dispatch<float>(p, g, w, stream);
}

MSEL_BOUNDS_TAKER(take_bounds_cplx_bwd)

}  // namespace msel
