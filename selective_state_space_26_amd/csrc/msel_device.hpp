// msel_device.hpp -- device-side building blocks of the gfx950 selective scan.
//
// * fp32 transcendentals as single CDNA instructions (v_exp_f32 is 2^x, v_log_f32 is log2).
// * bf16 <-> fp32 conversion (bf16 is the upper half of an fp32 word; stores round to
//   nearest even with the gfx950 v_cvt_pk_bf16_f32 instruction).
// * Row loads/stores of K consecutive time steps per lane, vectorized when the row is 16-byte
//   aligned and fully in range, element-wise with bounds checks otherwise.
// * Affine-pair scans over a 64-lane wavefront.  The recurrence h_t = a_t h_{t-1} + b_t is
//   affine in h, so pairs compose associatively, (a2,b2) o (a1,b1) = (a2 a1, a2 b1 + b2);
//   that is what makes the work-efficient parallel scan of page 1 possible.  The forward scan
//   uses DPP row_shr 1/2/4/8 inside 16-lane rows and row_bcast 15/31 across rows; the
//   reverse (suffix) scan uses DPP row_shl inside rows and ds_swizzle / readlane across rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msel {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// log(1 + e^x) = max(x, 0) + log1p(e^{-|x|}).  log1p(e) for e in (0, 1] uses the classic
// correction log1p(e) = log(w) * e / (w - 1), w = 1 + e rounded, which cancels the rounding
// of w; when w rounds to 1, log1p(e) = e to working precision.
__device__ __forceinline__ float softplus_f(float x) {
    float e = exp2_hw(-fabsf(x) * kLog2e);
    float w = 1.0f + e;
    float l = (w == 1.0f) ? e : log2_hw(w) * kLn2 * (e * rcp_hw(w - 1.0f));
    return fmaxf(x, 0.0f) + l;
}

__device__ __forceinline__ float sigmoid_f(float x) { return rcp_hw(1.0f + exp2_hw(-x * kLog2e)); }

// ---------------------------------------------------------------------------------------
// dtype traits: float rows, or bf16 rows stored as uint16_t.

struct bf16_t {
    uint16_t bits;
};

template <typename T> struct Elem;

template <> struct Elem<float> {
    static constexpr int kPerVec = 4;  // elements per 16-byte vector
    __device__ static float load1(const float* p) { return *p; }
    __device__ static void store1(float* p, float v) { *p = v; }
};

template <> struct Elem<bf16_t> {
    static constexpr int kPerVec = 8;
    __device__ static float load1(const bf16_t* p) {
        return __uint_as_float(static_cast<uint32_t>(p->bits) << 16);
    }
    __device__ static void store1(bf16_t* p, float v) {
        __bf16 h = static_cast<__bf16>(v);
        p->bits = __builtin_bit_cast(uint16_t, h);
    }
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    bf2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// Unpack one 16-byte vector of T into fp32 values v[j*kPerVec ...].
template <typename T, int K>
__device__ __forceinline__ void unpack_vec(u32x4 w, int j, float (&v)[K]) {
    if constexpr (sizeof(T) == 4) {
        v[4 * j + 0] = __uint_as_float(w.x);
        v[4 * j + 1] = __uint_as_float(w.y);
        v[4 * j + 2] = __uint_as_float(w.z);
        v[4 * j + 3] = __uint_as_float(w.w);
    } else {
        v[8 * j + 0] = bf16lo(w.x);
        v[8 * j + 1] = bf16hi(w.x);
        v[8 * j + 2] = bf16lo(w.y);
        v[8 * j + 3] = bf16hi(w.y);
        v[8 * j + 4] = bf16lo(w.z);
        v[8 * j + 5] = bf16hi(w.z);
        v[8 * j + 6] = bf16lo(w.w);
        v[8 * j + 7] = bf16hi(w.w);
    }
}

// Buffer resource of one row of L elements (the pointer is wave-uniform).  Buffer accesses
// are range-checked by the hardware: a load past the end returns zeros and a store past the
// end is dropped, so no branch or select is needed at the ragged end (an if/else around loads
// would make the second arm wait for the first arm's loads).  The third descriptor dword is
// the gfx9 raw-buffer format (32-bit data, no swizzle).
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const T* row, int L) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(row), 0,
                                             L * static_cast<int>(sizeof(T)), 0x00020000);
}

// One 16-byte vector of a VEC row holding steps [t, t + width): with the row 16-byte aligned,
// L a multiple of the vector width and t a multiple of it, the vector is wholly in range or
// wholly past the end (then it reads zeros).  NT: non-temporal (streaming) hint.
template <typename T, bool NT>
__device__ __forceinline__ u32x4 load_vec(const T* __restrict__ row, int t, int L) {
    return __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(row_rsrc(row, L), t * static_cast<int>(sizeof(T)),
                                                     0, NT ? 2 : 0));
}

// Load K consecutive elements row[t0 .. t0+K) as fp32; out-of-range elements read 0.
// VEC: the row base is 16-byte aligned, L is a multiple of the vector width and t0 a
// multiple of K.  Streaming (non-temporal) loads: for rows read once.
template <typename T, int K, bool VEC>
__device__ __forceinline__ void load_k(const T* __restrict__ row, int t0, int L, float (&v)[K],
                                       float /*fill: always 0*/) {
    static_assert(K % Elem<T>::kPerVec == 0, "K must be a whole number of 16-byte vectors");
    constexpr int VW = Elem<T>::kPerVec;
    if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < K / VW; ++j) unpack_vec<T, K>(load_vec<T, true>(row, t0 + j * VW, L), j, v);
    } else {
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = (t0 + k < L) ? Elem<T>::load1(row + t0 + k) : 0.0f;
    }
}

// Same as load_k but through the normal (cached) path, for rows that are read again.
template <typename T, int K, bool VEC>
__device__ __forceinline__ void load_k_cached(const T* __restrict__ row, int t0, int L,
                                              float (&v)[K]) {
    constexpr int VW = Elem<T>::kPerVec;
    if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < K / VW; ++j) unpack_vec<T, K>(load_vec<T, false>(row, t0 + j * VW, L), j, v);
    } else {
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = (t0 + k < L) ? Elem<T>::load1(row + t0 + k) : 0.0f;
    }
}

// Store K consecutive elements row[t0 .. t0+K) (out-of-range ones are dropped).  NT: the
// non-temporal (streaming) hint, for rows nothing reads soon.
template <typename T, int K, bool VEC, bool NT = true>
__device__ __forceinline__ void store_k(T* __restrict__ row, int t0, int L, const float (&v)[K]) {
    constexpr int VW = Elem<T>::kPerVec;
    if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < K / VW; ++j) {
            const int t = t0 + j * VW;  // a vector wholly past the end is dropped
            u32x4 w;
            if constexpr (sizeof(T) == 4) {
                w.x = __float_as_uint(v[4 * j + 0]);
                w.y = __float_as_uint(v[4 * j + 1]);
                w.z = __float_as_uint(v[4 * j + 2]);
                w.w = __float_as_uint(v[4 * j + 3]);
            } else {
                w.x = pack_bf16(v[8 * j + 0], v[8 * j + 1]);
                w.y = pack_bf16(v[8 * j + 2], v[8 * j + 3]);
                w.z = pack_bf16(v[8 * j + 4], v[8 * j + 5]);
                w.w = pack_bf16(v[8 * j + 6], v[8 * j + 7]);
            }
            __builtin_amdgcn_raw_buffer_store_b128(w, row_rsrc(row, L),
                                                   t * static_cast<int>(sizeof(T)), 0, NT ? 2 : 0);
        }
    } else {
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (t0 + k < L) Elem<T>::store1(row + t0 + k, v[k]);
    }
}

// Raw (still packed) rows: loads issued early and unpacked to fp32 only when used, so that
// the next state's B/C rows can be in flight while the current state is computed.
template <typename T, int K>
struct Raw {
    static constexpr int kVecs = K * static_cast<int>(sizeof(T)) / 16;
    u32x4 v[kVecs];
};

template <typename T, int K, bool VEC>
__device__ __forceinline__ void load_raw(const T* __restrict__ row, int t0, int L, Raw<T, K>& r) {
    constexpr int VW = Elem<T>::kPerVec;
    if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < Raw<T, K>::kVecs; ++j) r.v[j] = load_vec<T, false>(row, t0 + j * VW, L);
    } else {
#pragma unroll
        for (int j = 0; j < Raw<T, K>::kVecs; ++j) {
            uint32_t wds[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (sizeof(T) == 4) {
                    const int t = t0 + 4 * j + q;
                    wds[q] = (t < L) ? __float_as_uint(reinterpret_cast<const float*>(row)[t]) : 0u;
                } else {
                    const int t = t0 + 8 * j + 2 * q;
                    const uint16_t* h = reinterpret_cast<const uint16_t*>(row);
                    const uint32_t lo = (t < L) ? h[t] : 0u;
                    const uint32_t hi = (t + 1 < L) ? h[t + 1] : 0u;
                    wds[q] = lo | (hi << 16);
                }
            }
            r.v[j] = u32x4{wds[0], wds[1], wds[2], wds[3]};
        }
    }
}

template <typename T, int K>
__device__ __forceinline__ void unpack(const Raw<T, K>& r, float (&v)[K]) {
#pragma unroll
    for (int j = 0; j < Raw<T, K>::kVecs; ++j) unpack_vec<T, K>(r.v[j], j, v);
}

// ---------------------------------------------------------------------------------------
// Cross-lane moves.

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float old, float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                 __builtin_bit_cast(int, v), CTRL,
                                                                 ROW_MASK, 0xf, false));
}

// DPP controls (GFX9 encoding).
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowShl1 = 0x101, kRowShl2 = 0x102, kRowShl4 = 0x104, kRowShl8 = 0x108;
constexpr int kWaveShr1 = 0x138, kWaveShl1 = 0x130;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

__device__ __forceinline__ float readlane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
// Lane `lane` of the result is v, the other lanes keep old (lane is wave-uniform).
__device__ __forceinline__ float writelane(float v, int lane, float old) {
    return (static_cast<int>(__lane_id()) == lane) ? v : old;
}

// One Hillis-Steele step: element l absorbs element l-s (which precedes it in time).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void fwd_step(float& P, float& S) {
    float Pp = dpp<CTRL, ROW_MASK>(1.0f, P);
    float Sp = dpp<CTRL, ROW_MASK>(0.0f, S);
    S = fmaf(P, Sp, S);
    P = P * Pp;
}

// Inclusive scan over the 64 lanes of a wave, lane 0 first in time:
// (P_l, S_l) <- (P_l,S_l) o (P_{l-1},S_{l-1}) o ... o (P_0,S_0).
__device__ __forceinline__ void wave_scan_fwd(float& P, float& S) {
    fwd_step<kRowShr1, 0xf>(P, S);
    fwd_step<kRowShr2, 0xf>(P, S);
    fwd_step<kRowShr4, 0xf>(P, S);
    fwd_step<kRowShr8, 0xf>(P, S);
    fwd_step<kRowBcast15, 0xa>(P, S);
    fwd_step<kRowBcast31, 0xc>(P, S);
}

// Exclusive version of an inclusive forward scan: lane l gets lane l-1's value, lane 0 the
// identity (1, 0).
__device__ __forceinline__ void wave_shift_fwd(float P, float S, float& Pex, float& Sex) {
    Pex = dpp<kWaveShr1, 0xf>(1.0f, P);
    Sex = dpp<kWaveShr1, 0xf>(0.0f, S);
}

// One reverse step: element l absorbs element l+s (which follows it in time), for the
// backward recurrence g_t = e_t g_{t+1} + c_t: (P_l,S_l) <- (P_l, S_l) o' (P_{l+s}, S_{l+s})
// meaning g_l_in = P_{l+s} x + S_{l+s} is fed into lane l: S_l += P_l S_{l+s}, P_l *= P_{l+s}.
template <int CTRL>
__device__ __forceinline__ void rev_step(float& P, float& S) {
    float Pp = dpp<CTRL, 0xf>(1.0f, P);
    float Sp = dpp<CTRL, 0xf>(0.0f, S);
    S = fmaf(P, Sp, S);
    P = P * Pp;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Inclusive suffix scan over 64 lanes, lane 63 last in time: lane l ends with the composition
// of lanes l..63 (lane 63 applied first).
__device__ __forceinline__ void wave_scan_rev(float& P, float& S) {
    rev_step<kRowShl1>(P, S);
    rev_step<kRowShl2>(P, S);
    rev_step<kRowShl4>(P, S);
    rev_step<kRowShl8>(P, S);
    const int lane = lane_id();
    // rows: lanes 0-15 absorb lane 16's row total, lanes 32-47 absorb lane 48's.
    // ds_swizzle bit mode within 32-lane halves: and_mask 0, or_mask 16 -> every lane reads
    // lane 16 of its half.
    {
        constexpr int pat = (0x00) | (0x10 << 5);
        float Pp = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, P), pat));
        float Sp = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, S), pat));
        bool take = (lane & 16) == 0;
        Pp = take ? Pp : 1.0f;
        Sp = take ? Sp : 0.0f;
        S = fmaf(P, Sp, S);
        P = P * Pp;
    }
    // lanes 0-31 absorb lane 32's total (the suffix of lanes 32..63).
    {
        float Pp = readlane(P, 32);
        float Sp = readlane(S, 32);
        bool take = lane < 32;
        Pp = take ? Pp : 1.0f;
        Sp = take ? Sp : 0.0f;
        S = fmaf(P, Sp, S);
        P = P * Pp;
    }
}

// Exclusive suffix: lane l gets lane l+1's inclusive suffix, lane 63 the identity.
__device__ __forceinline__ void wave_shift_rev(float P, float S, float& Pex, float& Sex) {
    Pex = dpp<kWaveShl1, 0xf>(1.0f, P);
    Sex = dpp<kWaveShl1, 0xf>(0.0f, S);
}

// Sum over the 64 lanes; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<kRowShr1, 0xf>(0.0f, v);
    v += dpp<kRowShr2, 0xf>(0.0f, v);
    v += dpp<kRowShr4, 0xf>(0.0f, v);
    v += dpp<kRowShr8, 0xf>(0.0f, v);
    v += dpp<kRowBcast15, 0xa>(0.0f, v);
    v += dpp<kRowBcast31, 0xc>(0.0f, v);
    return readlane(v, 63);
}


// ---------------------------------------------------------------------------------------
// Scans with the DPP move fused into the arithmetic.  With bound_ctrl off, a lane whose DPP
// source does not exist (or whose row is masked off) is not written at all, which is exactly
// the identity element of the affine composition, so no identity values have to be set up:
//   v_fmac_f32_dpp S, S, P  ->  S_l = S_{src} * P_l + S_l
//   v_mul_f32_dpp  P, P, P  ->  P_l = P_{src} * P_l
// (the fmac reads P before the mul overwrites it).  GFX9 needs two wait states between a VALU
// write of a VGPR and a DPP read of it; the s_nop after every level (and before the first)
// provides them.

#define MSEL_FWD_LEVEL(CTRL, RMASK)                                              \
    "v_fmac_f32_dpp %[S], %[S], %[P] " CTRL " row_mask:" RMASK " bank_mask:0xf\n" \
    "v_mul_f32_dpp %[P], %[P], %[P] " CTRL " row_mask:" RMASK " bank_mask:0xf\n"  \
    "s_nop 1\n"

// Inclusive forward scan over the 64 lanes of a wave (lane 0 first in time).
__device__ __forceinline__ void scan_fwd_fused(float& P, float& S) {
    asm volatile("s_nop 1\n"
                 MSEL_FWD_LEVEL("row_shr:1", "0xf")
                 MSEL_FWD_LEVEL("row_shr:2", "0xf")
                 MSEL_FWD_LEVEL("row_shr:4", "0xf")
                 MSEL_FWD_LEVEL("row_shr:8", "0xf")
                 MSEL_FWD_LEVEL("row_bcast:15", "0xa")
                 MSEL_FWD_LEVEL("row_bcast:31", "0xc")
                 : [P] "+v"(P), [S] "+v"(S));
}

// Inclusive suffix scan over the 64 lanes (lane 63 last in time): the row levels are fused
// DPP row_shl; the two cross-row levels use ds_swizzle and readlane.
__device__ __forceinline__ void scan_rev_fused(float& P, float& S) {
    asm volatile("s_nop 1\n"
                 MSEL_FWD_LEVEL("row_shl:1", "0xf")
                 MSEL_FWD_LEVEL("row_shl:2", "0xf")
                 MSEL_FWD_LEVEL("row_shl:4", "0xf")
                 MSEL_FWD_LEVEL("row_shl:8", "0xf")
                 : [P] "+v"(P), [S] "+v"(S));
    const int lane = lane_id();
    {
        constexpr int pat = (0x10 << 5);  // every lane of a 32-lane half reads its lane 16
        const float Pp = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, P), pat));
        const float Sp = __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, S), pat));
        const bool take = (lane & 16) == 0;
        S = take ? fmaf(P, Sp, S) : S;
        P = take ? P * Pp : P;
    }
    {
        const float Pp = readlane(P, 32);
        const float Sp = readlane(S, 32);
        const bool take = lane < 32;
        S = take ? fmaf(P, Sp, S) : S;
        P = take ? P * Pp : P;
    }
}

// The forward scan of (P, S) and the row levels of the suffix scan of (Pr, Sr) in one
// instruction stream.  The two are independent, so each one's DPP reads come at least two
// instructions after the other's writes and the row levels need no wait states; only the two
// cross-row levels of the forward scan keep theirs.  On return (P, S) is the full inclusive
// scan over the wave and (Pr, Sr) the suffix scan within each 16-lane row (finish it with
// rev_rows_apply).
__device__ __forceinline__ void scan_fwd_and_rev_rows(float& P, float& S, float& Pr, float& Sr) {
#define MSEL_PAIR_LEVEL(CF, CR)                                                         \
    "v_fmac_f32_dpp %[S], %[S], %[P] " CF " row_mask:0xf bank_mask:0xf\n"              \
    "v_mul_f32_dpp %[P], %[P], %[P] " CF " row_mask:0xf bank_mask:0xf\n"               \
    "v_fmac_f32_dpp %[Sr], %[Sr], %[Pr] " CR " row_mask:0xf bank_mask:0xf\n"           \
    "v_mul_f32_dpp %[Pr], %[Pr], %[Pr] " CR " row_mask:0xf bank_mask:0xf\n"
    asm volatile("s_nop 1\n"
                 MSEL_PAIR_LEVEL("row_shr:1", "row_shl:1")
                 MSEL_PAIR_LEVEL("row_shr:2", "row_shl:2")
                 MSEL_PAIR_LEVEL("row_shr:4", "row_shl:4")
                 MSEL_PAIR_LEVEL("row_shr:8", "row_shl:8")
                 MSEL_FWD_LEVEL("row_bcast:15", "0xa")
                 MSEL_FWD_LEVEL("row_bcast:31", "0xc")
                 : [P] "+v"(P), [S] "+v"(S), [Pr] "+v"(Pr), [Sr] "+v"(Sr));
#undef MSEL_PAIR_LEVEL
}

// Row levels (16-lane rows) of four independent scans in one instruction stream: (P1, S1) and
// (P2, S2) forward (row_shr), (Q1, R1) and (Q2, R2) suffix (row_shl).  Each DPP read comes at
// least three instructions after the write of its source, so no wait states are needed.
__device__ __forceinline__ void scan_rows4(float& P1, float& S1, float& Q1, float& R1, float& P2,
                                           float& S2, float& Q2, float& R2) {
#define MSEL_ROW4(CF, CR)                                                            \
    "v_fmac_f32_dpp %[S1], %[S1], %[P1] " CF " row_mask:0xf bank_mask:0xf\n"         \
    "v_mul_f32_dpp %[P1], %[P1], %[P1] " CF " row_mask:0xf bank_mask:0xf\n"          \
    "v_fmac_f32_dpp %[R1], %[R1], %[Q1] " CR " row_mask:0xf bank_mask:0xf\n"         \
    "v_mul_f32_dpp %[Q1], %[Q1], %[Q1] " CR " row_mask:0xf bank_mask:0xf\n"          \
    "v_fmac_f32_dpp %[S2], %[S2], %[P2] " CF " row_mask:0xf bank_mask:0xf\n"         \
    "v_mul_f32_dpp %[P2], %[P2], %[P2] " CF " row_mask:0xf bank_mask:0xf\n"          \
    "v_fmac_f32_dpp %[R2], %[R2], %[Q2] " CR " row_mask:0xf bank_mask:0xf\n"         \
    "v_mul_f32_dpp %[Q2], %[Q2], %[Q2] " CR " row_mask:0xf bank_mask:0xf\n"
    asm volatile("s_nop 1\n"
                 MSEL_ROW4("row_shr:1", "row_shl:1")
                 MSEL_ROW4("row_shr:2", "row_shl:2")
                 MSEL_ROW4("row_shr:4", "row_shl:4")
                 MSEL_ROW4("row_shr:8", "row_shl:8")
                 : [P1] "+v"(P1), [S1] "+v"(S1), [Q1] "+v"(Q1), [R1] "+v"(R1),
                   [P2] "+v"(P2), [S2] "+v"(S2), [Q2] "+v"(Q2), [R2] "+v"(R2));
#undef MSEL_ROW4
}

// Row levels of two independent suffix scans (row_shl), interleaved; the DPP reads come two
// instructions after the writes of their sources, which is the wait the hardware needs.
__device__ __forceinline__ void scan_rows2_rev(float& Q1, float& R1, float& Q2, float& R2) {
#define MSEL_ROW2(CR)                                                                \
    "v_fmac_f32_dpp %[R1], %[R1], %[Q1] " CR " row_mask:0xf bank_mask:0xf\n"         \
    "v_mul_f32_dpp %[Q1], %[Q1], %[Q1] " CR " row_mask:0xf bank_mask:0xf\n"          \
    "v_fmac_f32_dpp %[R2], %[R2], %[Q2] " CR " row_mask:0xf bank_mask:0xf\n"         \
    "v_mul_f32_dpp %[Q2], %[Q2], %[Q2] " CR " row_mask:0xf bank_mask:0xf\n"
    asm volatile("s_nop 1\n"
                 MSEL_ROW2("row_shl:1")
                 MSEL_ROW2("row_shl:2")
                 MSEL_ROW2("row_shl:4")
                 MSEL_ROW2("row_shl:8")
                 : [Q1] "+v"(Q1), [R1] "+v"(R1), [Q2] "+v"(Q2), [R2] "+v"(R2));
#undef MSEL_ROW2
}

// Row levels of four independent suffix scans (row_shl), interleaved.
__device__ __forceinline__ void scan_rows4_rev(float& Q1, float& R1, float& Q2, float& R2,
                                               float& Q3, float& R3, float& Q4, float& R4) {
#define MSEL_ROWR4(CR)                                                               \
    "v_fmac_f32_dpp %[R1], %[R1], %[Q1] " CR " row_mask:0xf bank_mask:0xf\n"         \
    "v_mul_f32_dpp %[Q1], %[Q1], %[Q1] " CR " row_mask:0xf bank_mask:0xf\n"          \
    "v_fmac_f32_dpp %[R2], %[R2], %[Q2] " CR " row_mask:0xf bank_mask:0xf\n"         \
    "v_mul_f32_dpp %[Q2], %[Q2], %[Q2] " CR " row_mask:0xf bank_mask:0xf\n"          \
    "v_fmac_f32_dpp %[R3], %[R3], %[Q3] " CR " row_mask:0xf bank_mask:0xf\n"         \
    "v_mul_f32_dpp %[Q3], %[Q3], %[Q3] " CR " row_mask:0xf bank_mask:0xf\n"          \
    "v_fmac_f32_dpp %[R4], %[R4], %[Q4] " CR " row_mask:0xf bank_mask:0xf\n"         \
    "v_mul_f32_dpp %[Q4], %[Q4], %[Q4] " CR " row_mask:0xf bank_mask:0xf\n"
    asm volatile("s_nop 1\n"
                 MSEL_ROWR4("row_shl:1")
                 MSEL_ROWR4("row_shl:2")
                 MSEL_ROWR4("row_shl:4")
                 MSEL_ROWR4("row_shl:8")
                 : [Q1] "+v"(Q1), [R1] "+v"(R1), [Q2] "+v"(Q2), [R2] "+v"(R2),
                   [Q3] "+v"(Q3), [R3] "+v"(R3), [Q4] "+v"(Q4), [R4] "+v"(R4));
#undef MSEL_ROWR4
}

// Totals of scans whose row levels are done (wave-uniform results):
//  forward: the composition of all 64 lanes, from the last lane of each row;
//  suffix:  the composition of all 64 lanes, from the first lane of each row.
// Only the S part is returned (the end state from a zero start, resp. the value at lane 0
// from a zero carry).
__device__ __forceinline__ float fwd_rows_total(float P, float S) {
    float t = readlane(S, 15);
    t = fmaf(readlane(P, 31), t, readlane(S, 31));
    t = fmaf(readlane(P, 47), t, readlane(S, 47));
    return fmaf(readlane(P, 63), t, readlane(S, 63));
}
__device__ __forceinline__ float rev_rows_total(float P, float S) {
    float t = readlane(S, 48);
    t = fmaf(readlane(P, 32), t, readlane(S, 32));
    t = fmaf(readlane(P, 16), t, readlane(S, 16));
    return fmaf(readlane(P, 0), t, readlane(S, 0));
}

// Finishes a suffix scan whose row levels are done: (P, S) of lane l compose lanes l..15 of
// its row.  `carry` is the value entering from beyond lane 63 (wave-uniform).  Returns, in
// every lane, the suffix composition of lanes l..63 applied to `carry`:
//   V_l = S_l + P_l R(row),  R(3) = carry,  R(r) = S_{16(r+1)} + P_{16(r+1)} R(r+1),
// read from the first lane of each following row (no LDS round trip).
__device__ __forceinline__ float rev_rows_apply(float P, float S, float carry) {
    const float R3 = carry;
    const float R2 = fmaf(readlane(P, 48), R3, readlane(S, 48));
    const float R1 = fmaf(readlane(P, 32), R2, readlane(S, 32));
    const float R0 = fmaf(readlane(P, 16), R1, readlane(S, 16));
    const int row = lane_id() >> 4;
    const float R = row == 0 ? R0 : (row == 1 ? R1 : (row == 2 ? R2 : R3));
    return fmaf(P, R, S);
}

// Sum over each group of four consecutive lanes (every lane of the group gets it).
__device__ __forceinline__ float quad_sum(float v) {
    v += dpp<0xB1, 0xf>(0.0f, v);  // quad_perm [1,0,3,2]
    v += dpp<0x4E, 0xf>(0.0f, v);  // quad_perm [2,3,0,1]
    return v;
}

// Lane l gets v of lane l-1; lane 0 gets `first`.
__device__ __forceinline__ float shift_up(float v, float first) {
    float r = first;
    asm volatile("s_nop 1\n"
                 "v_mov_b32_dpp %[r], %[v] wave_shr:1 row_mask:0xf bank_mask:0xf\n"
                 : [r] "+v"(r) : [v] "v"(v));
    return r;
}

// Lane l gets v of lane l+1; lane 63 gets `last`.
__device__ __forceinline__ float shift_down(float v, float last) {
    float r = last;
    asm volatile("s_nop 1\n"
                 "v_mov_b32_dpp %[r], %[v] wave_shl:1 row_mask:0xf bank_mask:0xf\n"
                 : [r] "+v"(r) : [v] "v"(v));
    return r;
}

// Sum over the 64 lanes with fused DPP adds; the total is returned in every lane.
__device__ __forceinline__ float wave_sum_fused(float v) {
    asm volatile("s_nop 1\n"
                 "v_add_f32_dpp %[v], %[v], %[v] row_shr:1 row_mask:0xf bank_mask:0xf\n"
                 "s_nop 1\n"
                 "v_add_f32_dpp %[v], %[v], %[v] row_shr:2 row_mask:0xf bank_mask:0xf\n"
                 "s_nop 1\n"
                 "v_add_f32_dpp %[v], %[v], %[v] row_shr:4 row_mask:0xf bank_mask:0xf\n"
                 "s_nop 1\n"
                 "v_add_f32_dpp %[v], %[v], %[v] row_shr:8 row_mask:0xf bank_mask:0xf\n"
                 "s_nop 1\n"
                 "v_add_f32_dpp %[v], %[v], %[v] row_bcast:15 row_mask:0xa bank_mask:0xf\n"
                 "s_nop 1\n"
                 "v_add_f32_dpp %[v], %[v], %[v] row_bcast:31 row_mask:0xc bank_mask:0xf\n"
                 "s_nop 1\n"
                 : [v] "+v"(v));
    return readlane(v, 63);
}

// Inclusive prefix sum over the 64 lanes (lane 0 first), fused DPP adds: a lane whose DPP
// source does not exist is not written, i.e. adds nothing.
__device__ __forceinline__ float wave_incl_sum(float v) {
    asm volatile("s_nop 1\n"
                 "v_add_f32_dpp %[v], %[v], %[v] row_shr:1 row_mask:0xf bank_mask:0xf\n"
                 "s_nop 1\n"
                 "v_add_f32_dpp %[v], %[v], %[v] row_shr:2 row_mask:0xf bank_mask:0xf\n"
                 "s_nop 1\n"
                 "v_add_f32_dpp %[v], %[v], %[v] row_shr:4 row_mask:0xf bank_mask:0xf\n"
                 "s_nop 1\n"
                 "v_add_f32_dpp %[v], %[v], %[v] row_shr:8 row_mask:0xf bank_mask:0xf\n"
                 "s_nop 1\n"
                 "v_add_f32_dpp %[v], %[v], %[v] row_bcast:15 row_mask:0xa bank_mask:0xf\n"
                 "s_nop 1\n"
                 "v_add_f32_dpp %[v], %[v], %[v] row_bcast:31 row_mask:0xc bank_mask:0xf\n"
                 : [v] "+v"(v));
    return v;
}

// Four independent 64-lane sums, interleaved so that no wait states are needed; lane 63 of
// each result holds the total (returned wave-uniform).
__device__ __forceinline__ void wave_sum4(float& a, float& b, float& c, float& d) {
#define MSEL_SUM4(CTRL, RMASK)                                                       \
    "v_add_f32_dpp %[a], %[a], %[a] " CTRL " row_mask:" RMASK " bank_mask:0xf\n"     \
    "v_add_f32_dpp %[b], %[b], %[b] " CTRL " row_mask:" RMASK " bank_mask:0xf\n"     \
    "v_add_f32_dpp %[c], %[c], %[c] " CTRL " row_mask:" RMASK " bank_mask:0xf\n"     \
    "v_add_f32_dpp %[d], %[d], %[d] " CTRL " row_mask:" RMASK " bank_mask:0xf\n"
    asm volatile("s_nop 1\n"
                 MSEL_SUM4("row_shr:1", "0xf")
                 MSEL_SUM4("row_shr:2", "0xf")
                 MSEL_SUM4("row_shr:4", "0xf")
                 MSEL_SUM4("row_shr:8", "0xf")
                 MSEL_SUM4("row_bcast:15", "0xa")
                 MSEL_SUM4("row_bcast:31", "0xc")
                 : [a] "+v"(a), [b] "+v"(b), [c] "+v"(c), [d] "+v"(d));
#undef MSEL_SUM4
    a = readlane(a, 63);
    b = readlane(b, 63);
    c = readlane(c, 63);
    d = readlane(d, 63);
}

}  // namespace msel
