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
//  3. gradient kernel: one workgroup per (batch, chunk, range of channels) with one wavefront
//     per state pair.  A wavefront keeps its pair's B and C rows of the chunk, and its dB and
//     dC sums over the workgroup's channels, in registers; per channel it rebuilds the states
//     (lane chains + complex affine DPP scan from H_c) and the adjoints (reverse lane chains +
//     complex suffix scan from G_c), and forms every term.  The per-token sums over pairs (for
//     du, dDelta and the gated y) meet in LDS.
#include "msel_device.hpp"
#include "msel_kernels.hpp"

namespace msel {

namespace {

constexpr float kInv2Pi = 0.15915494309189535f;
constexpr int kK = kChunk / 64;  // steps per lane
constexpr int kMaxPairs = 8;

struct CWork {
    const float* H;  // [B*D*nch*N]: chunk-start states (the forward's chunk_states)
    float* G;        // [B*D*nch*N]: per chunk the local adjoint, then the adjoint carry
    float* sdt;      // [B*D*nch]: sum of Delta over the chunk
    float* dfirst;   // [B*D*nch]: Delta at the chunk's first step
    int c0;          // first chunk summarised: chunk 0's summary feeds only dh0, so it is
                     // skipped (c0 = 1) when dh0 is not asked for
};

__device__ __forceinline__ float sin_rev(float r) {
    return __builtin_amdgcn_sinf(__builtin_amdgcn_fractf(r));
}
__device__ __forceinline__ float cos_rev(float r) {
    return __builtin_amdgcn_cosf(__builtin_amdgcn_fractf(r));
}

// (P, S) <- (P Q, P T + S) with (Q, T) from the DPP source lane, identity where there is none.
template <int CTRL, int RM>
__device__ __forceinline__ void cplx_level(float& Pr, float& Pi, float& Sr, float& Si) {
    const float qr = dpp<CTRL, RM>(1.0f, Pr);
    const float qi = dpp<CTRL, RM>(0.0f, Pi);
    const float tr = dpp<CTRL, RM>(0.0f, Sr);
    const float ti = dpp<CTRL, RM>(0.0f, Si);
    const float nSr = fmaf(Pr, tr, fmaf(-Pi, ti, Sr));
    const float nSi = fmaf(Pr, ti, fmaf(Pi, tr, Si));
    const float nPr = fmaf(Pr, qr, -Pi * qi);
    const float nPi = fmaf(Pr, qi, Pi * qr);
    Pr = nPr;
    Pi = nPi;
    Sr = nSr;
    Si = nSi;
}

// Inclusive prefix composition over the 64 lanes (lane 0 applied first).
__device__ __forceinline__ void cplx_scan_fwd(float& Pr, float& Pi, float& Sr, float& Si) {
    cplx_level<kRowShr1, 0xf>(Pr, Pi, Sr, Si);
    cplx_level<kRowShr2, 0xf>(Pr, Pi, Sr, Si);
    cplx_level<kRowShr4, 0xf>(Pr, Pi, Sr, Si);
    cplx_level<kRowShr8, 0xf>(Pr, Pi, Sr, Si);
    cplx_level<kRowBcast15, 0xa>(Pr, Pi, Sr, Si);
    cplx_level<kRowBcast31, 0xc>(Pr, Pi, Sr, Si);
}

// Inclusive suffix composition inside each 16-lane row (the row's last lane applied first):
// afterwards lane 16r holds the composition of its whole row.
__device__ __forceinline__ void cplx_scan_rev_rows(float& Pr, float& Pi, float& Sr, float& Si) {
    cplx_level<kRowShl1, 0xf>(Pr, Pi, Sr, Si);
    cplx_level<kRowShl2, 0xf>(Pr, Pi, Sr, Si);
    cplx_level<kRowShl4, 0xf>(Pr, Pi, Sr, Si);
    cplx_level<kRowShl8, 0xf>(Pr, Pi, Sr, Si);
}

__device__ __forceinline__ void cmul(float ar, float ai, float br, float bi, float& r, float& i) {
    r = fmaf(ar, br, -ai * bi);
    i = fmaf(ar, bi, ai * br);
}

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
    const size_t ch = static_cast<size_t>(b) * p.D + d;
    const size_t row = ch * L;
    const int t0 = c * kChunk + lane * K;
    const float bias = p.bias ? p.bias[d] : 0.0f;

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
    // E_t: sum of Delta over the chunk's steps 1..t
    float E[K];
    float run = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        run += dt[k];
        E[k] = run;
    }
    const float incl = wave_incl_sum(run);
    const float before = incl - run;                 // Delta of the lanes before this one
    const float first = readlane(dt[0], 0);          // Delta at the chunk's first step
    const float total = readlane(incl, 63);
#pragma unroll
    for (int k = 0; k < K; ++k) E[k] += before - first;

    const T* __restrict__ Cg = static_cast<const T*>(p.Cm) + static_cast<size_t>(b) * N * L;
    const float* Ad = p.A + static_cast<size_t>(d) * N;
    float outv = 0.0f;  // lane n: component n of the summary
    for (int n = 0; n < N; n += 4) {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // (re, im) of pairs n/2 and n/2 + 1
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int m = n + 2 * q;
            if (m >= N) break;
            const float Ar = Ad[m] * kLog2e, Ai = Ad[m + 1] * kInv2Pi;
            float cr[K], ci[K];
            load_k_cached<T, K, VEC>(Cg + static_cast<size_t>(m) * L, t0, L, cr);
            load_k_cached<T, K, VEC>(Cg + static_cast<size_t>(m + 1) * L, t0, L, ci);
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
    const size_t base = ch * nch + c;
    if (lane < N) w.G[base * N + lane] = outv;
    if (lane == 0) {
        w.sdt[base] = total;
        w.dfirst[base] = first;
    }
}

// ---------------------------------------------------------------------------------------
// 2. link

__global__ __launch_bounds__(256) void cplx_link_kernel(ScanParams p, GradParams g, CWork w) {
    const int J = p.N / 2;
    const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= static_cast<long long>(p.B) * p.D * J) return;
    const long long ch = i / J;
    const int j = static_cast<int>(i - ch * J);
    const int d = static_cast<int>(ch % p.D);
    const int nch = p.nchunks;
    const float Ar = p.A[static_cast<size_t>(d) * p.N + 2 * j] * kLog2e;
    const float Ai = p.A[static_cast<size_t>(d) * p.N + 2 * j + 1] * kInv2Pi;
    float Gr = 0.0f, Gi = 0.0f;
    for (int c = nch - 1; c >= w.c0; --c) {
        const size_t base = static_cast<size_t>(ch) * nch + c;
        float* slot = w.G + base * p.N + 2 * j;
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
        float* slot = w.G + static_cast<size_t>(ch) * nch * p.N + 2 * j;
        slot[0] = Gr;
        slot[1] = Gi;
    }
    if (g.dh0 != nullptr) {
        g.dh0[static_cast<size_t>(ch) * p.N + 2 * j] = Gr;
        g.dh0[static_cast<size_t>(ch) * p.N + 2 * j + 1] = Gi;
    }
}

// ---------------------------------------------------------------------------------------
// 3. gradient kernel

// LDS: per-token partial sums [3][pair][kChunk] (sum_n Re(conj G) B, the dDelta terms of a,
// and y for the gate), then the finished per-token outputs [3][kChunk]; a lane's step k sits at
// k * 64 + lane, so that the 64 lanes touch consecutive words.
constexpr size_t cplx_main_lds_bytes() { return (3 * kMaxPairs + 3) * kChunk * sizeof(float); }

template <typename T, bool VEC, bool HAS_Z, bool SOFTPLUS>
__global__ __launch_bounds__(64 * kMaxPairs) void cplx_main_kernel(ScanParams p, GradParams g,
                                                                   CWork w, int per_wg) {
    constexpr int K = kK;
    __shared__ float red[3 * kMaxPairs * kChunk];
    __shared__ float fin[3 * kChunk];
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));  // pair
    const int J = p.N / 2;
    const int b = blockIdx.z;
    const int c = blockIdx.y;
    const int N = p.N, L = p.L, nch = p.nchunks;
    const int d0 = blockIdx.x * per_wg;
    const int d1 = min(p.D, d0 + per_wg);
    const int t0 = c * kChunk + lane * K;
    const int n0 = 2 * wv;

    // this pair's B and C for the chunk (zero past the end), kept for all channels
    float Br[K], Bi[K], Cr[K], Ci[K];
    {
        const T* Bg = static_cast<const T*>(p.Bm) + static_cast<size_t>(b) * N * L;
        const T* Cg = static_cast<const T*>(p.Cm) + static_cast<size_t>(b) * N * L;
        load_k_cached<T, K, VEC>(Bg + static_cast<size_t>(n0) * L, t0, L, Br);
        load_k_cached<T, K, VEC>(Bg + static_cast<size_t>(n0 + 1) * L, t0, L, Bi);
        load_k_cached<T, K, VEC>(Cg + static_cast<size_t>(n0) * L, t0, L, Cr);
        load_k_cached<T, K, VEC>(Cg + static_cast<size_t>(n0 + 1) * L, t0, L, Ci);
    }
    float dBr[K], dBi[K], dCr[K], dCi[K];
#pragma unroll
    for (int k = 0; k < K; ++k) dBr[k] = dBi[k] = dCr[k] = dCi[k] = 0.0f;

    // the next channel's rows (packed) and chunk values, fetched while one is computed:
    // lane parity picks (Re, Im) of H_c and G_c, so these are vector loads
    Raw<T, K> ru, rd, rg, rz;
    float nH = 0.0f, nG = 0.0f;
    auto fetch = [&](int dn) {
        const size_t rown = (static_cast<size_t>(b) * p.D + dn) * L;
        load_raw<T, K, VEC>(static_cast<const T*>(p.u) + rown, t0, L, ru);
        load_raw<T, K, VEC>(static_cast<const T*>(p.delta) + rown, t0, L, rd);
        load_raw<T, K, VEC>(static_cast<const T*>(g.dout) + rown, t0, L, rg);
        if constexpr (HAS_Z) load_raw<T, K, VEC>(static_cast<const T*>(p.z) + rown, t0, L, rz);
        const size_t hgn = ((static_cast<size_t>(b) * p.D + dn) * nch + c) * N + n0 + (lane & 1);
        nH = w.H[hgn];
        nG = w.G[hgn];
    };
    if (d0 < d1) fetch(d0);

    for (int d = d0; d < d1; ++d) {
        const size_t ch = static_cast<size_t>(b) * p.D + d;
        const size_t row = ch * L;
        const float bias = p.bias ? p.bias[d] : 0.0f;
        const float Dd = p.Dv ? p.Dv[d] : 0.0f;
        const float ArRaw = p.A[static_cast<size_t>(d) * N + n0];
        const float AiRaw = p.A[static_cast<size_t>(d) * N + n0 + 1];
        const float Ar = ArRaw * kLog2e, Ai = AiRaw * kInv2Pi;
        // this channel's u, dout and z stay packed for the epilogue
        const Raw<T, K> cu = ru, cg = rg, cz = rz;
        float dt[K], dtu[K], dy[K];
        float sum_dt = 0.0f;
        {
            float uu[K], dd[K], go[K];
            unpack<T, K>(ru, uu);
            unpack<T, K>(rd, dd);
            unpack<T, K>(rg, go);
            float zz[HAS_Z ? K : 1];
            if constexpr (HAS_Z) unpack<T, K>(rz, zz);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float x = dd[k] + bias;
                const float v = SOFTPLUS ? softplus_f(x) : x;
                dt[k] = (t0 + k < L) ? v : 0.0f;
                dtu[k] = dt[k] * uu[k];
                dy[k] = HAS_Z ? go[k] * zz[k] * sigmoid_f(zz[k]) : go[k];
                sum_dt += dt[k];
            }
        }
        const float Hr = readlane(nH, 0), Hi = readlane(nH, 1);
        const float Gr = readlane(nG, 0), Gi = readlane(nG, 1);
        if (d + 1 < d1) fetch(d + 1);

        // pass 1: transitions, the lane chain of states from zero, the lane transitions
        float ar[K], ai[K];
        float hr = 0.0f, hi = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float e = exp2_hw(dt[k] * Ar);
            const float r = dt[k] * Ai;
            ar[k] = e * cos_rev(r);
            ai[k] = e * sin_rev(r);
            const float nr = fmaf(ar[k], hr, fmaf(-ai[k], hi, dtu[k] * Br[k]));
            hi = fmaf(ai[k], hr, fmaf(ar[k], hi, dtu[k] * Bi[k]));
            hr = nr;
        }
        const float eP = exp2_hw(sum_dt * Ar), rP = sum_dt * Ai;
        float Pr = eP * cos_rev(rP), Pi = eP * sin_rev(rP), Sr = hr, Si = hi;
        cplx_scan_fwd(Pr, Pi, Sr, Si);
        float Qr, Qi;  // the state after the lane's last step
        {
            float tr, ti;
            cmul(Pr, Pi, Hr, Hi, tr, ti);
            Qr = tr + Sr;
            Qi = ti + Si;
        }
        const float hin_r = shift_up(Qr, Hr), hin_i = shift_up(Qi, Hi);

        // the adjoint: lane chain from a zero input on the right,
        // g_k = dy C_k + conj(a_{k+1}) g_{k+1}
        float gr = dy[K - 1] * Cr[K - 1], gi = dy[K - 1] * Ci[K - 1];
#pragma unroll
        for (int k = K - 2; k >= 0; --k) {
            const float xr = ar[k + 1], xi = ai[k + 1];
            const float tr = fmaf(xr, gr, xi * gi), ti = fmaf(xr, gi, -xi * gr);
            gr = fmaf(dy[k], Cr[k], tr);
            gi = fmaf(dy[k], Ci[k], ti);
        }
        // lane map from the adjoint arriving on the right (already carried into the lane's
        // last step) to the one leaving on the left: Q(x) = conj(a_0) (g_0 + P x) with
        // P = conj(a_1 ... a_{K-1}) = conj(exp(A (sum_dt - dt_0)))
        float Rr, Ri, Tr, Ti;
        {
            const float s1 = sum_dt - dt[0];
            const float e1 = exp2_hw(s1 * Ar), r1 = s1 * Ai;
            const float p1r = e1 * cos_rev(r1), p1i = -e1 * sin_rev(r1);
            const float c0r = ar[0], c0i = -ai[0];
            cmul(c0r, c0i, p1r, p1i, Rr, Ri);
            cmul(c0r, c0i, gr, gi, Tr, Ti);
        }
        cplx_scan_rev_rows(Rr, Ri, Tr, Ti);
        // the adjoint arriving on the right of each row, from G_c through the rows above
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
        float vr, vi;  // the adjoint leaving this lane on the left
        {
            float tr, ti;
            cmul(Rr, Ri, er, ei, tr, ti);
            vr = tr + Tr;
            vi = ti + Ti;
        }
        // the adjoint arriving on this lane's right: the next lane's, G_c for lane 63
        const float gin_r = shift_down(vr, Gr), gin_i = shift_down(vi, Gi);

        // pass 2: states, y, dC
        float hsr[K], hsi[K];
        float ypart[K];
        hr = hin_r;
        hi = hin_i;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float nr = fmaf(ar[k], hr, fmaf(-ai[k], hi, dtu[k] * Br[k]));
            hi = fmaf(ai[k], hr, fmaf(ar[k], hi, dtu[k] * Bi[k]));
            hr = nr;
            hsr[k] = hr;
            hsi[k] = hi;
            ypart[k] = fmaf(Cr[k], hr, Ci[k] * hi);
            dCr[k] = fmaf(dy[k], hr, dCr[k]);
            dCi[k] = fmaf(dy[k], hi, dCi[k]);
        }
        // reverse pass: the adjoint at every step and the gradient terms
        float sB[K], sgA[K];
        float dAr = 0.0f, dAi = 0.0f;
        gr = gin_r;
        gi = gin_i;
#pragma unroll
        for (int k = K - 1; k >= 0; --k) {
            if (k < K - 1) {
                const float xr = ar[k + 1], xi = ai[k + 1];
                const float tr = fmaf(xr, gr, xi * gi), ti = fmaf(xr, gi, -xi * gr);
                gr = tr;
                gi = ti;
            }
            gr = fmaf(dy[k], Cr[k], gr);
            gi = fmaf(dy[k], Ci[k], gi);
            dBr[k] = fmaf(gr, dtu[k], dBr[k]);
            dBi[k] = fmaf(gi, dtu[k], dBi[k]);
            sB[k] = fmaf(gr, Br[k], gi * Bi[k]);
            const float pr = (k == 0) ? hin_r : hsr[k - 1];
            const float pi = (k == 0) ? hin_i : hsi[k - 1];
            float ahr, ahi;
            cmul(ar[k], ai[k], pr, pi, ahr, ahi);
            // X = conj(g) a h_prev
            const float Xr = fmaf(gr, ahr, gi * ahi), Xi = fmaf(gr, ahi, -gi * ahr);
            sgA[k] = fmaf(ArRaw, Xr, -AiRaw * Xi);
            dAr = fmaf(dt[k], Xr, dAr);
            dAi = fmaf(-dt[k], Xi, dAi);
        }
        // dA[d, 2j], dA[d, 2j+1]
        {
            float z0 = 0.0f, z1 = 0.0f;
            wave_sum4(dAr, dAi, z0, z1);
            if (g.dA != nullptr && lane < 2)
                unsafeAtomicAdd(g.dA + static_cast<size_t>(d) * N + n0 + lane, lane == 0 ? dAr : dAi);
        }
        // per-token sums over the pairs
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int tok = k * 64 + lane;  // k-major: conflict-free LDS rows
            red[(0 * kMaxPairs + wv) * kChunk + tok] = sB[k];
            red[(1 * kMaxPairs + wv) * kChunk + tok] = sgA[k];
            if constexpr (HAS_Z) red[(2 * kMaxPairs + wv) * kChunk + tok] = ypart[k];
        }
        __syncthreads();
        // wave wv finishes the tokens k = wv, wv + J, ... of every lane
        {
            float uu[K];
            unpack<T, K>(cu, uu);
            float zz[HAS_Z ? K : 1], go[HAS_Z ? K : 1];
            if constexpr (HAS_Z) {
                unpack<T, K>(cz, zz);
                unpack<T, K>(cg, go);
            }
#pragma unroll
            for (int k = 0; k < K; ++k) {
                if ((k % J) != (wv % J) || k < wv) continue;
                const int tok = k * 64 + lane;  // k-major: conflict-free LDS rows
                float sb = 0.0f, sg = 0.0f, yv = 0.0f;
                for (int q = 0; q < J; ++q) {
                    sb += red[(0 * kMaxPairs + q) * kChunk + tok];
                    sg += red[(1 * kMaxPairs + q) * kChunk + tok];
                    if constexpr (HAS_Z) yv += red[(2 * kMaxPairs + q) * kChunk + tok];
                }
                const float dsp = SOFTPLUS ? 1.0f - exp2_hw(-dt[k] * kLog2e) : 1.0f;
                fin[0 * kChunk + tok] = fmaf(sb, dt[k], dy[k] * Dd);        // du
                fin[1 * kChunk + tok] = fmaf(sb, uu[k], sg) * dsp;          // ddelta
                if constexpr (HAS_Z) {
                    yv = fmaf(Dd, uu[k], yv);
                    const float s = sigmoid_f(zz[k]);
                    fin[2 * kChunk + tok] = go[k] * s * fmaf(zz[k], 1.0f - s, 1.0f) * yv;  // dz
                }
            }
        }
        __syncthreads();
        // wave (d mod J) stores the channel's du, ddelta, dz and adds dD, dbias
        if (wv == d % J) {
            float o1[K], o2[K], o3[HAS_Z ? K : 1];
            float db = 0.0f, dDp = 0.0f;
            float uu[K];
            unpack<T, K>(cu, uu);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int tok = k * 64 + lane;  // k-major: conflict-free LDS rows
                o1[k] = fin[0 * kChunk + tok];
                o2[k] = fin[1 * kChunk + tok];
                if constexpr (HAS_Z) o3[k] = fin[2 * kChunk + tok];
                db += (t0 + k < L) ? o2[k] : 0.0f;
                dDp = fmaf(dy[k], uu[k], dDp);
            }
            store_k<T, K, VEC>(static_cast<T*>(g.du) + row, t0, L, o1);
            store_k<T, K, VEC>(static_cast<T*>(g.ddelta) + row, t0, L, o2);
            if constexpr (HAS_Z) store_k<T, K, VEC>(static_cast<T*>(g.dz) + row, t0, L, o3);
            float z0 = 0.0f, z1 = 0.0f;
            wave_sum4(db, dDp, z0, z1);
            if (lane == 0 && g.dbias != nullptr) unsafeAtomicAdd(g.dbias + d, db);
            if (lane == 1 && g.dD != nullptr) unsafeAtomicAdd(g.dD + d, dDp);
        }
    }
    // this workgroup's share of dB and dC for the pair
    if (t0 < L) {
        const size_t o = (static_cast<size_t>(b) * N + n0) * L;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (t0 + k >= L) break;
            if (g.dB != nullptr) {
                unsafeAtomicAdd(g.dB + o + t0 + k, dBr[k]);
                unsafeAtomicAdd(g.dB + o + L + t0 + k, dBi[k]);
            }
            if (g.dC != nullptr) {
                unsafeAtomicAdd(g.dC + o + t0 + k, dCr[k]);
                unsafeAtomicAdd(g.dC + o + L + t0 + k, dCi[k]);
            }
        }
    }
}

int cplx_compute_units() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    return cus;
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
    hipLaunchKernelGGL(cplx_link_kernel, dim3(static_cast<unsigned>((links + 255) / 256)),
                       dim3(256), 0, s, p, g, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // channels per workgroup: about two workgroups per compute unit over (batch, chunk,
    // channel ranges), so that the dB / dC flush is amortised over many channels
    static const int cus = cplx_compute_units();
    const long long slots = static_cast<long long>(p.B) * p.nchunks;
    long long per = (static_cast<long long>(p.D) * slots + 2LL * cus - 1) / (2LL * cus);
    if (per < 1) per = 1;
    if (per > p.D) per = p.D;
    const int cg = static_cast<int>((p.D + per - 1) / per);
    hipLaunchKernelGGL((cplx_main_kernel<T, VEC, HAS_Z, SP>), dim3(cg, p.nchunks, p.B),
                       dim3(64 * (p.N / 2)), 0, s, p, g, w, static_cast<int>(per));
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

static_assert(cplx_main_lds_bytes() <= 64 * 1024, "static LDS of the complex gradient kernel");

}  // namespace

hipError_t launch_scan_cplx_bwd(const ScanParams& p, const GradParams& g,
                                const float* chunk_states, void* workspace, bool bf16,
                                hipStream_t stream) {
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
    return bf16 ? cplx_bwd_dispatch<bf16_t>(p, g, w, stream)
                : cplx_bwd_dispatch<float>(p, g, w, stream);
}

}  // namespace msel
